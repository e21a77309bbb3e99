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
#include "topk.h"

namespace nvfp4 {
namespace {

constexpr int kMaxExperts = 1024;
constexpr int kMaxPerLane = kMaxExperts / kWave;  // 16 logits per lane
constexpr int kTopkThreads = 256;
constexpr int kRouteDecodeThreads = 64 * (kMaxRouteExperts / 64);   // 8 waves per token

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
__device__ void wave_topk(const LogitSrc &src, int64_t t, int E, int k, int renormalize,
                          int32_t *ids, float *weights, int32_t *ids_copy) {
  const int lane = threadIdx.x & 63;
  float v[kMaxPerLane];
  const int per_lane = (E + 63) / 64;
  load_logits(src, t, E, lane, v);
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

// One workgroup of 8 waves per token (more than 256 experts: the
// workgroup-wide ranking, block_topk8).
__global__ __launch_bounds__(kRouteDecodeThreads) void topk_block_kernel(
    const LogitSrc logits, int64_t T, int E, int k, int renormalize, int32_t *ids,
    float *weights) {
  __shared__ uint64_t cand[kMaxRouteExperts / 8];
  __shared__ float lgt[kMaxRouteExperts];
  const int64_t t = blockIdx.x;
  int id;
  float wgt;
  block_topk8(logits, t, E, k, renormalize, cand, lgt, id, wgt);
  const int lane = threadIdx.x & 63;
  if ((threadIdx.x >> 6) == 0 && lane < k) {
    ids[t * k + lane] = id;
    weights[t * k + lane] = wgt;
  }
}

// One wavefront per token.
__global__ __launch_bounds__(kTopkThreads) void topk_merge_kernel(
    const LogitSrc logits, int64_t T, int E, int k, int renormalize, int32_t *ids,
    float *weights) {
  const int64_t t = (int64_t)blockIdx.x * (kTopkThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  wave_topk_merge(logits, t, E, k, renormalize, ids + t * k, weights + t * k, nullptr);
}

// One wavefront per token.
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    const LogitSrc logits, int64_t T, int E, int k, int renormalize, int32_t *ids,
    float *weights) {
  const int64_t t = (int64_t)blockIdx.x * (kTopkThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  wave_topk(logits, t, E, k, renormalize, ids + t * k, weights + t * k, nullptr);
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
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
  // inclusive prefix sum over the 64 lanes (row shifts, then row broadcasts)
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);   // row_bcast:31
  (void)lane;
  return x;
}

// Pairs whose id lies outside 0..E-1 are dropped: they take no position, the
// expert offsets count only the kept pairs (offsets[E] = kept), and the
// positions kept .. P-1 of sorted_pairs hold -1.

// Sum of the per-wave totals of a workgroup scan (read after its barrier).
__device__ __forceinline__ int64_t block_total(const int32_t *wave_tot, int nwaves) {
  int64_t total = 0;
  for (int w = 0; w < nwaves; ++w) total += wave_tot[w];
  return total;
}

// -1 into positions kept .. P-1 of sorted_pairs (the workgroup's threads).
__device__ __forceinline__ void fill_dropped(int32_t *sorted_pairs, int64_t kept, int64_t P) {
  for (int64_t q = kept + threadIdx.x; q < P; q += blockDim.x) sorted_pairs[q] = -1;
}

// One-chunk case (T <= 32 W tokens): no separate counting pass.  The pairs
// set their token bits; then one wave per expert turns the expert's W words
// into running popcounts with a wave scan (the expert's total comes with
// it), a scan over the experts gives the offsets, and each pair's position
// is its expert's offset + the tokens before its word + the set bits below
// it in the word.  Four barriers, no counter contention.
__device__ void permute_block_one_chunk(const int32_t *ids, int64_t T, int E, int k, int W,
                                        int32_t *offsets, int32_t *sorted_pairs, PermuteLds &L) {
  uint32_t *bitmap = L.bitmap;
  uint16_t *prefix = L.prefix;
  int32_t *cnt = L.cnt, *off = L.off, *wave_tot = L.wave_tot;
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63, wave = tid >> 6;
  const int nwaves = nthr >> 6;
  const int64_t P = T * k;
  for (int i = tid; i < E * W; i += nthr) bitmap[i] = 0u;
  __syncthreads();
  // pairs in batches of 8 per thread, so eight id loads are in flight at once
  constexpr int kBatchIds = 8;
  for (int64_t p0 = tid; p0 < P; p0 += (int64_t)nthr * kBatchIds) {
    int e8[kBatchIds];
#pragma unroll
    for (int u = 0; u < kBatchIds; ++u) {
      const int64_t p = p0 + (int64_t)u * nthr;
      e8[u] = p < P ? ids[p] : -1;
    }
#pragma unroll
    for (int u = 0; u < kBatchIds; ++u) {
      const int64_t p = p0 + (int64_t)u * nthr;
      if (p < P && (unsigned)e8[u] < (unsigned)E) {   // (other ids: dropped pairs)
        const int64_t t = p / k;
        atomicOr(&bitmap[e8[u] * W + (int)(t >> 5)], 1u << (t & 31));
      }
    }
  }
  __syncthreads();
  // per expert: exclusive running popcount over its words (a thread per
  // expert for short rows of words, a wave scan per expert for long ones)
  if (W <= 32) {
    for (int e = tid; e < E; e += nthr) {
      int run = 0;
      for (int w = 0; w < W; ++w) {
        prefix[e * W + w] = (uint16_t)run;
        run += __popc(bitmap[e * W + w]);
      }
      cnt[e] = run;
    }
  } else {
    for (int e = wave; e < E; e += nwaves) {
      int run = 0;
      for (int w0 = 0; w0 < W; w0 += 64) {
        const int w = w0 + lane;
        const int c = w < W ? __popc(bitmap[e * W + w]) : 0;
        const int incl = wave_incl_scan(c, lane);
        if (w < W) prefix[e * W + w] = (uint16_t)(run + incl - c);
        run += __builtin_amdgcn_readlane(incl, 63);
      }
      if (lane == 0) cnt[e] = run;
    }
  }
  __syncthreads();
  // exclusive scan of the expert totals (thread tid owns ept experts)
  {
    const int ept = (E + nthr - 1) / nthr;
    const int e0 = tid * ept;
    int c = 0;
    for (int i = 0; i < ept; ++i)
      if (e0 + i < E) c += cnt[e0 + i];
    const int incl = wave_incl_scan(c, lane);
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
  }
  const int64_t kept = block_total(L.wave_tot, nwaves);
  if (tid == 0) offsets[E] = (int32_t)kept;
  fill_dropped(sorted_pairs, kept, P);
  __syncthreads();
  for (int64_t p0 = tid; p0 < P; p0 += (int64_t)nthr * kBatchIds) {
    int e8[kBatchIds];
#pragma unroll
    for (int u = 0; u < kBatchIds; ++u) {
      const int64_t p = p0 + (int64_t)u * nthr;
      e8[u] = p < P ? ids[p] : -1;
    }
#pragma unroll
    for (int u = 0; u < kBatchIds; ++u) {
      const int64_t p = p0 + (int64_t)u * nthr;
      if (p < P && (unsigned)e8[u] < (unsigned)E) {
        const int e = e8[u];
        const int64_t t = p / k;
        const int w = (int)(t >> 5);
        const uint32_t below = bitmap[e * W + w] & ((1u << (t & 31)) - 1u);
        sorted_pairs[off[e] + prefix[e * W + w] + __popc(below)] = (int32_t)p;
      }
    }
  }
}

__device__ void permute_block(const int32_t *ids, int64_t T, int E, int k, int W,
                              int32_t *offsets, int32_t *sorted_pairs, PermuteLds &L) {
  if (T <= (int64_t)W * 32) {
    permute_block_one_chunk(ids, T, E, k, W, offsets, sorted_pairs, L);
    return;
  }
  uint32_t *bitmap = L.bitmap;
  uint16_t *prefix = L.prefix;
  int32_t *cnt = L.cnt, *off = L.off, *base = L.base, *chunk_cnt = L.chunk_cnt;
  int32_t *wave_tot = L.wave_tot;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int64_t P = T * k;

  for (int e = tid; e < E; e += nthr) { cnt[e] = 0; base[e] = 0; }
  __syncthreads();
  for (int64_t p = tid; p < P; p += nthr) {
    const int e = ids[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);   // (other ids: dropped pairs)
  }
  __syncthreads();

  // exclusive scan of cnt over E <= 1024 experts: thread tid owns the ept
  // consecutive experts tid * ept ..
  {
    const int ept = (E + nthr - 1) / nthr;
    const int e0 = tid * ept;
    int c = 0;
    for (int i = 0; i < ept; ++i)
      if (e0 + i < E) c += cnt[e0 + i];
    const int lane = tid & 63, wave = tid >> 6;
    const int incl = wave_incl_scan(c, lane);
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
  }
  const int64_t kept = block_total(wave_tot, nthr >> 6);
  if (tid == 0) offsets[E] = (int32_t)kept;
  fill_dropped(sorted_pairs, kept, P);
  __syncthreads();

  const int64_t chunk_tokens = (int64_t)W * 32;
  for (int64_t t0 = 0; t0 < T; t0 += chunk_tokens) {
    const int64_t t1 = t0 + chunk_tokens < T ? t0 + chunk_tokens : T;
    for (int i = tid; i < E * W; i += nthr) bitmap[i] = 0u;
    __syncthreads();
    for (int64_t p = t0 * k + tid; p < t1 * k; p += nthr) {
      const int e = ids[p];
      if ((unsigned)e >= (unsigned)E) continue;   // dropped pair
      const int64_t tl = p / k - t0;
      atomicOr(&bitmap[e * W + (int)(tl >> 5)], 1u << (tl & 31));
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
      if ((unsigned)e >= (unsigned)E) continue;   // dropped pair
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

// Permutation of a larger batch spread over workgroups by expert: workgroup
// g owns experts [g epw, (g + 1) epw).  It reads every pair's id twice (L2
// hits).  The first pass counts the pairs whose expert lies below its range
// (the offset of its first expert) and marks its own pairs' tokens in a
// bitmap per own expert; running popcounts over each bitmap then give every
// own expert its count and, with the count below, its offset; the second
// pass sends own pair p (expert e, token t) to offsets[e] + (tokens of e
// before t), the stable counting-sort position.  Each offset is written by
// exactly one workgroup; the last also writes offsets[E].
constexpr int kSplitThreads = 1024;
constexpr int kSplitWords = 8192;     // own experts x words per expert
constexpr int kSplitMaxEpw = 64;
constexpr int kSplitGroups = 128;     // target workgroup count

__global__ __launch_bounds__(kSplitThreads) void permute_split_kernel(
    const int32_t *ids, int64_t T, int E, int k, int epw, int W, int32_t *offsets,
    int32_t *sorted_pairs) {
  __shared__ uint32_t bitmap[kSplitWords];
  __shared__ uint32_t prefix[kSplitWords];
  __shared__ int32_t own_cnt[kSplitMaxEpw];
  __shared__ int32_t own_off[kSplitMaxEpw];
  __shared__ int32_t wave_below[kSplitThreads / 64];
  __shared__ int32_t kept_lds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthr = blockDim.x, nwaves = nthr >> 6;
  const int e_lo = blockIdx.x * epw;
  const int e_hi = e_lo + epw < E ? e_lo + epw : E;
  const int nown = e_hi - e_lo;
  const int64_t P = T * k;
  for (int i = tid; i < nown * W; i += nthr) bitmap[i] = 0u;
  __syncthreads();

  // pass 1: pairs below the range, own tokens into the bitmaps
  constexpr int kBatchIds = 8;
  int below = 0;
  for (int64_t p0 = tid; p0 < P; p0 += (int64_t)nthr * kBatchIds) {
    int e8[kBatchIds];
#pragma unroll
    for (int u = 0; u < kBatchIds; ++u) {
      const int64_t p = p0 + (int64_t)u * nthr;
      const int v = p < P ? ids[p] : E;
      e8[u] = (unsigned)v < (unsigned)E ? v : E;   // (dropped pairs: above every expert)
    }
#pragma unroll
    for (int u = 0; u < kBatchIds; ++u) {
      const int64_t p = p0 + (int64_t)u * nthr;
      const int e = e8[u];
      below += e < e_lo;
      if (e >= e_lo && e < e_hi) {
        const int64_t t = p / k;
        atomicOr(&bitmap[(e - e_lo) * W + (int)(t >> 5)], 1u << (t & 31));
      }
    }
  }
  {
    const int incl = wave_incl_scan(below, lane);
    if (lane == 63) wave_below[wave] = incl;
  }
  __syncthreads();
  // running popcounts of each own expert's words (one wave per expert)
  for (int ee = wave; ee < nown; ee += nwaves) {
    int run = 0;
    for (int w0 = 0; w0 < W; w0 += 64) {
      const int w = w0 + lane;
      const int c = w < W ? __popc(bitmap[ee * W + w]) : 0;
      const int incl = wave_incl_scan(c, lane);
      if (w < W) prefix[ee * W + w] = (uint32_t)(run + incl - c);
      run += __builtin_amdgcn_readlane(incl, 63);
    }
    if (lane == 0) own_cnt[ee] = run;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < nwaves; ++w) run += wave_below[w];
    for (int ee = 0; ee < nown; ++ee) {
      own_off[ee] = run;
      offsets[e_lo + ee] = run;
      run += own_cnt[ee];
    }
    if (e_hi == E) {   // the last group: every kept pair lies below its end
      offsets[E] = run;
      kept_lds = run;
    }
  }
  __syncthreads();
  if (e_hi == E) fill_dropped(sorted_pairs, kept_lds, P);

  // pass 2: own pairs to their positions
  for (int64_t p0 = tid; p0 < P; p0 += (int64_t)nthr * kBatchIds) {
    int e8[kBatchIds];
#pragma unroll
    for (int u = 0; u < kBatchIds; ++u) {
      const int64_t p = p0 + (int64_t)u * nthr;
      e8[u] = p < P ? ids[p] : E;
    }
#pragma unroll
    for (int u = 0; u < kBatchIds; ++u) {
      const int64_t p = p0 + (int64_t)u * nthr;
      const int e = e8[u];
      if (e >= e_lo && e < e_hi) {   // (a dropped pair's id never lies in 0..E-1)
        const int ee = e - e_lo;
        const int64_t t = p / k;
        const int w = (int)(t >> 5);
        const uint32_t lower = bitmap[ee * W + w] & ((1u << (t & 31)) - 1u);
        sorted_pairs[own_off[ee] + (int)prefix[ee * W + w] + __popc(lower)] = (int32_t)p;
      }
    }
  }
}

// Permutation of a decode-sized batch (T k <= 256 pairs, E <= 1024), one
// workgroup of 256 threads: expert counts by LDS atomics, one wave scans
// them into the offsets, and pair p (expert e) goes to offsets[e] plus the
// number of earlier pairs with expert e, counted directly from the ids in
// LDS: the stable counting-sort result in three barriers.
__global__ __launch_bounds__(256) void permute_small_kernel(const int32_t *ids, int64_t T, int E,
                                                            int k, int32_t *offsets,
                                                            int32_t *sorted_pairs) {
  __shared__ int32_t ids_lds[kSmallPairs];
  __shared__ int32_t cnt[kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63;
  const int P = (int)T * k;
  for (int e = tid; e < E; e += 256) cnt[e] = 0;
  __shared__ int32_t kept_lds;
  int my_e = -1;   // -1: no pair, or a dropped one (id outside 0..E-1)
  if (tid < P) {
    const int v = ids[tid];
    my_e = (unsigned)v < (unsigned)E ? v : -1;
    ids_lds[tid] = my_e;
  }
  __syncthreads();
  if (my_e >= 0) atomicAdd(&cnt[my_e], 1);
  __syncthreads();
  if (tid < 64) {   // exclusive scan: lane l owns experts l * per .. (l + 1) * per - 1
    const int per = (E + 63) / 64;
    const int e0 = lane * per;
    int local = 0;
    for (int i = 0; i < per; ++i)
      if (e0 + i < E) local += cnt[e0 + i];
    const int incl = wave_incl_scan(local, lane);
    int run = incl - local;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < E) {
        const int c = cnt[e];
        cnt[e] = run;   // now the expert's first position
        offsets[e] = run;
        run += c;
      }
    }
    if (lane == 63) {   // the last lane's run ends after every kept pair
      offsets[E] = run;
      kept_lds = run;
    }
  }
  __syncthreads();
  if (tid >= kept_lds && tid < P) sorted_pairs[tid] = -1;
  if (my_e >= 0) {
    int before = 0;
    for (int q = 0; q < tid; ++q) before += ids_lds[q] == my_e;
    sorted_pairs[cnt[my_e] + before] = tid;
  }
}

// Decode-sized routing in one launch (T k <= 256 pairs, E <= 512, k <= 8):
// one workgroup of 8 waves per token (tokens spread over CUs) takes the
// top-k (block_topk8) and its wave 0 publishes ids and weights, then takes
// a ticket from a counter in the caller's workspace; the workgroup holding
// the last ticket, which therefore sees every token's ids, resets the
// counter and its wave 0 builds the permutation (wave_permute_small,
// bit-sliced matching).  The ids are written and read as device-scope
// (relaxed agent) atomics, performed at the device's coherence point past
// the per-XCD L2s, and the wave waits for its stores to complete before
// taking its ticket: this orders them before the last workgroup's reads
// without the whole-L2 write-back and invalidate that release and acquire
// fences cost.
__global__ __launch_bounds__(kRouteDecodeThreads) void route_decode_kernel(
    const LogitSrc logits, int64_t T, int E, int k, int renormalize, int32_t *ids,
    float *weights, int32_t *offsets, int32_t *sorted_pairs, uint32_t *ticket) {
  __shared__ int32_t first[kMaxRouteExperts];
  __shared__ uint64_t cand[kMaxRouteExperts / 8];
  __shared__ float lgt[kMaxRouteExperts];
  __shared__ uint32_t last;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int t = blockIdx.x;
  int id;
  float wgt;
  block_topk8(logits, t, E, k, renormalize, cand, lgt, id, wgt);
  if (wave == 0) {
    if (lane < k) {
      __hip_atomic_store(ids + (int64_t)t * k + lane, id, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      weights[(int64_t)t * k + lane] = wgt;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's ids stores complete
    uint32_t mine = 0;
    if (lane == 0)
      mine = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    mine = __builtin_amdgcn_readfirstlane(mine);
    if (lane == 0) {
      last = mine == (uint32_t)T - 1 ? 1u : 0u;
      if (mine == (uint32_t)T - 1)
        __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  if (!last) return;   // (uniform: the whole workgroup)
  wave_permute_small(
      [&](int p) { return __hip_atomic_load(ids + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); },
      (int)T * k, E, offsets, sorted_pairs, first, wave == 0);
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

// Zeroes the ticket word of a routing workspace (a kernel rather than a
// memset, so the call may sit in a captured graph).
__global__ __launch_bounds__(64) void ticket_reset_kernel(uint32_t *ticket) {
  if (threadIdx.x == 0) *ticket = 0u;
}

}  // namespace

hipError_t launch_ticket_reset(uint32_t *ticket, hipStream_t s) {
  launch_kernel(ticket_reset_kernel, dim3(1), dim3(64), 0, s, ticket);
  return hipGetLastError();
}

bool route_decode_supported(int64_t T, int E, int k) {
  return T * k <= kSmallPairs && E <= 512 && k <= 8;
}

hipError_t launch_route(const LogitSrc &logits, int64_t T, int E, int k, int renormalize,
                        int32_t *ids, float *weights, int32_t *offsets, int32_t *sorted_pairs,
                        uint32_t *ticket, hipStream_t s) {
  if (ticket && route_decode_supported(T, E, k)) {
    launch_kernel(route_decode_kernel, dim3((unsigned)T), dim3(kRouteDecodeThreads), 0, s, logits,
                  T, E, k, renormalize, ids, weights, offsets, sorted_pairs, ticket);
    return hipGetLastError();
  }
  hipError_t e = launch_topk(logits, T, E, k, renormalize, ids, weights, s);
  if (e != hipSuccess) return e;
  return launch_permute(ids, T, E, k, offsets, sorted_pairs, s);
}

hipError_t launch_topk(const LogitSrc &logits, int64_t T, int E, int k, int renormalize,
                       int32_t *ids, float *weights, hipStream_t s) {
  // over 256 experts one 8-wave workgroup per token (block_topk8); else one
  // wavefront per token, four per workgroup, so a decode batch spreads over
  // several CUs (one wave per SIMD) instead of sharing one
  const int64_t blocks = (T + 3) / 4;
  if (E > 256 && E <= 512 && k <= 8)
    launch_kernel(topk_block_kernel, dim3((unsigned)T), dim3(kRouteDecodeThreads), 0, s, logits,
                  T, E, k, renormalize, ids, weights);
  else if (E <= 512 && k <= 8)
    launch_kernel(topk_merge_kernel, dim3((unsigned)blocks), dim3(kTopkThreads), 0, s, logits, T,
                  E, k, renormalize, ids, weights);
  else
    launch_kernel(topk_kernel, dim3((unsigned)blocks), dim3(kTopkThreads), 0, s, logits, T, E, k,
                  renormalize, ids, weights);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t *ids, int64_t T, int E, int k, int32_t *offsets,
                          int32_t *sorted_pairs, hipStream_t s) {
  const int W = permute_words(T, E);
  // permutation: one workgroup for a decode-sized batch, else spread over
  // workgroups by expert while each one's bitmaps fit in LDS
  if (T * k <= kSmallPairs) {
    launch_kernel(permute_small_kernel, dim3(1), dim3(256), 0, s, ids, T, E, k, offsets,
                  sorted_pairs);
    return hipGetLastError();
  }
  {
    const int64_t words = (T + 31) / 32;
    int64_t epw = (E + kSplitGroups - 1) / kSplitGroups;
    if (epw > kSplitMaxEpw) epw = kSplitMaxEpw;
    if (words * epw <= kSplitWords) {
      const int groups = (int)((E + epw - 1) / epw);
      launch_kernel(permute_split_kernel, dim3((unsigned)groups), dim3(kSplitThreads), 0, s, ids,
                    T, E, k, (int)epw, (int)words, offsets, sorted_pairs);
      return hipGetLastError();
    }
  }
  launch_kernel(permute_kernel, dim3(1), dim3(kPermThreads), 0, s, ids, T, E, k, W, offsets,
                sorted_pairs);
  return hipGetLastError();
}

}  // namespace nvfp4

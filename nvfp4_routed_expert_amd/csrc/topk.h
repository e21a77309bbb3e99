// Device-side top-k of one token's logits (the merge network) and the
// one-wavefront permutation of a decode-sized batch, shared by the routing
// kernels and the fused decode FFN, which routes its own token.
//
// The Flash-Next model routes every token to a few of its 512 MoE experts
// (Eider page, "Qwen3.8 Flash Next").  Selection compares the fp32 logits
// (ties to the lower expert index) and the permutation is the stable
// counting sort of the (token, slot) pairs by expert.
#pragma once

#include "common.h"
#include "kernels.h"

namespace nvfp4 {
namespace {

constexpr int kSmallPairs = 256;         // decode-sized batches: pairs
constexpr int kMaxRouteExperts = 512;    // ... and experts per token row

// Token t's logits at experts lane + 64 i (i < N; 0 past E): the part sums
// added in part order (at most kMaxLogitParts parts), then the bias; written
// to src.out when that is set.  Every load is issued before the first add
// and the stores come last, so a row costs one round trip.
template <int N>
__device__ __forceinline__ void load_logits(const LogitSrc &src, int64_t t, int E, int lane,
                                            float (&v)[N]) {
  const float *row = src.part + t * E;
  float p[N][kMaxLogitParts], b[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int e = lane + 64 * i;
    const bool ok = e < E;
#pragma unroll
    for (int s = 0; s < kMaxLogitParts; ++s)
      p[i][s] = (ok && s < src.parts) ? row[s * src.part_stride + e] : 0.0f;
    b[i] = (ok && src.bias) ? src.bias[e] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float x = p[i][0];
#pragma unroll
    for (int s = 1; s < kMaxLogitParts; ++s)
      if (s < src.parts) x += p[i][s];
    if (src.bias) x += b[i];
    v[i] = x;
  }
  if (src.out) {
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (lane + 64 * i < E) src.out[t * E + lane + 64 * i] = v[i];
  }
}

// ---- merge-network top-k (E <= 512, k <= 8) -------------------------------
//
// The round-by-round argmax above is a long dependent chain (k rounds of a
// six-level reduction).  For the common decode shapes this variant orders
// 64-bit keys instead: key = (order-preserving bits of the logit, complement
// of the index), so a larger key is a larger logit or, on equal logits, a
// lower index (the same order as `beats`; -0 is folded into +0 first).  Each
// lane sorts its 8 keys with a 19-comparator network, then six merge levels
// pair lanes (xor 1, xor 2, the mirrored lane in 8 and in 16 through DPP,
// then the other row and the other half through permlane swaps); a merge
// keeps the top 8 of both sorted lists (elementwise max against the
// partner's reversed list, then a bitonic clean-up).  Both partners compute
// the same list, so after the last level every lane holds the sorted top 8.

__device__ __forceinline__ uint64_t topk_key(float v, int e) {
  const uint32_t b = __float_as_uint(v + 0.0f);   // -0 -> +0
  const uint32_t m = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)m << 32) | (uint32_t)~(uint32_t)e;
}

// keep the larger key in x, the smaller in y
__device__ __forceinline__ void cas(uint64_t &x, uint64_t &y) {
  const bool sw = y > x;
  const uint64_t hi = sw ? y : x, lo = sw ? x : y;
  x = hi;
  y = lo;
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint32_t swap16_partner(uint32_t x, int lane) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return ((lane >> 4) & 1) ? (uint32_t)r[0] : (uint32_t)r[1];
}
__device__ __forceinline__ uint32_t swap32_partner(uint32_t x, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return lane >= 32 ? (uint32_t)r[0] : (uint32_t)r[1];
}

template <int LEVEL>
__device__ __forceinline__ uint64_t partner_key(uint64_t v, int lane) {
  if constexpr (LEVEL == 0) return dpp_u64<0xB1>(v);    // lane ^ 1
  if constexpr (LEVEL == 1) return dpp_u64<0x4E>(v);    // lane ^ 2
  if constexpr (LEVEL == 2) return dpp_u64<0x141>(v);   // 7 - i within 8
  if constexpr (LEVEL == 3) return dpp_u64<0x140>(v);   // 15 - i within 16
  if constexpr (LEVEL == 4)
    return ((uint64_t)swap16_partner((uint32_t)(v >> 32), lane) << 32) |
           swap16_partner((uint32_t)v, lane);
  return ((uint64_t)swap32_partner((uint32_t)(v >> 32), lane) << 32) |
         swap32_partner((uint32_t)v, lane);
}

template <int LEVEL>
__device__ __forceinline__ void merge_level(uint64_t (&c)[8], int lane) {
  uint64_t b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = partner_key<LEVEL>(c[i], lane);
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = c[i] > b[7 - i] ? c[i] : b[7 - i];
#pragma unroll
  for (int d = 4; d >= 1; d >>= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i & d) == 0) cas(c[i], c[i + d]);
}

[[maybe_unused]] __device__ void wave_topk_merge(const LogitSrc &src, int64_t t, int E, int k,
                                                int renormalize, int32_t *ids, float *weights,
                                                int32_t *ids_copy, bool device_scope_ids = false) {
  const int lane = threadIdx.x & 63;
  float v[8];
  uint64_t c[8];
  load_logits(src, t, E, lane, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = lane + 64 * i;
    c[i] = e < E ? topk_key(v[i], e) : 0ull;
  }
  constexpr int kNet[19][2] = {{0, 2}, {1, 3}, {4, 6}, {5, 7}, {0, 4}, {1, 5}, {2, 6},
                               {3, 7}, {0, 1}, {2, 3}, {4, 5}, {6, 7}, {2, 4}, {3, 5},
                               {1, 4}, {3, 6}, {1, 2}, {3, 4}, {5, 6}};
#pragma unroll
  for (int n = 0; n < 19; ++n) cas(c[kNet[n][0]], c[kNet[n][1]]);
  merge_level<0>(c, lane);
  merge_level<1>(c, lane);
  merge_level<2>(c, lane);
  merge_level<3>(c, lane);
  merge_level<4>(c, lane);
  merge_level<5>(c, lane);
  // lane j < k takes the j-th key
  uint64_t mine = c[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mine = lane == i ? c[i] : mine;
  const int my_idx = (int)~(uint32_t)mine;
  const uint32_t m = (uint32_t)(mine >> 32);
  const float my_val = __uint_as_float((m & 0x80000000u) ? (m & 0x7FFFFFFFu) : ~m);
  const float lmax = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_val), 0));
  const float ex = lane < k ? expf(my_val - lmax) : 0.0f;
  float denom;
  if (renormalize) {
    denom = wave_sum(ex);
  } else {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (lane + 64 * i < E) s += expf(v[i] - lmax);
    denom = wave_sum(s);
  }
  if (lane < k) {
    if (device_scope_ids)
      __hip_atomic_store(ids + lane, my_idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      ids[lane] = my_idx;
    weights[lane] = ex / denom;
    if (ids_copy) ids_copy[lane] = my_idx;
  }
}

// ---- cross-lane top 8 (one key per lane) -----------------------------------
//
// A bitonic network over the 64 lanes of a wave, one 64-bit key per lane
// (keys as above): groups of 8 lanes are sorted (flip steps at distance 2, 4
// and 8, each followed by half-cleaners), then sorted groups are merged in
// pairs keeping the larger half (the lower group's lanes take the max
// against the mirrored partner group, then half-cleaners at 4, 2, 1), with
// the partner group in the same 16-lane row, the other row of the half, and
// the other half.  Lanes 0..7 end with the wave's 8 largest keys in
// descending order (the other lanes hold leftovers).

// k against its partner p: the larger when keep_max, else the smaller
__device__ __forceinline__ uint64_t cx_key(uint64_t k, uint64_t p, bool keep_max) {
  const bool gt = p > k;
  return keep_max == gt ? p : k;
}
// lane ^ 4 within rows of 16 (row shifts by 4, the valid side chosen)
__device__ __forceinline__ uint64_t xor4_key(uint64_t v, int lane) {
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  const uint32_t lo_up = __builtin_amdgcn_update_dpp(0u, lo, 0x104, 0xF, 0xF, false);   // row_shl:4
  const uint32_t hi_up = __builtin_amdgcn_update_dpp(0u, hi, 0x104, 0xF, 0xF, false);
  const uint32_t lo_dn = __builtin_amdgcn_update_dpp(0u, lo, 0x114, 0xF, 0xF, false);   // row_shr:4
  const uint32_t hi_dn = __builtin_amdgcn_update_dpp(0u, hi, 0x114, 0xF, 0xF, false);
  const bool up = (lane & 4) == 0;   // partner is lane + 4
  return ((uint64_t)(up ? hi_up : hi_dn) << 32) | (up ? lo_up : lo_dn);
}
__device__ __forceinline__ uint64_t wave_top8_lanes(uint64_t key, int lane) {
  auto clean8 = [&](uint64_t v) {
    v = cx_key(v, xor4_key(v, lane), (lane & 4) == 0);
    v = cx_key(v, dpp_u64<0x4E>(v), (lane & 2) == 0);    // lane ^ 2
    return cx_key(v, dpp_u64<0xB1>(v), (lane & 1) == 0);  // lane ^ 1
  };
  key = cx_key(key, dpp_u64<0xB1>(key), (lane & 1) == 0);
  key = cx_key(key, dpp_u64<0x1B>(key), (lane & 3) < 2);     // 3 - i within 4
  key = cx_key(key, dpp_u64<0xB1>(key), (lane & 1) == 0);
  key = cx_key(key, dpp_u64<0x141>(key), (lane & 7) < 4);    // 7 - i within 8
  key = cx_key(key, dpp_u64<0x4E>(key), (lane & 2) == 0);
  key = cx_key(key, dpp_u64<0xB1>(key), (lane & 1) == 0);
  key = clean8(cx_key(key, dpp_u64<0x140>(key), (lane & 15) < 8));                // 15 - i
  key = clean8(cx_key(key, dpp_u64<0x141>(partner_key<4>(key, lane)), (lane & 16) == 0));
  key = clean8(cx_key(key, dpp_u64<0x141>(partner_key<5>(key, lane)), lane < 32));
  return key;
}

// Top-k (k <= 8) of token t's logits (E <= 512) by a workgroup of W waves,
// 64 W >= E, every wave of which calls it (it holds one barrier): waves
// 0..min(W, 8)-1 each rank 64 logits (the logits as load_logits forms
// them), wave 0 ranks their 8 best each and computes the weights with
// wave_topk_merge's arithmetic in the same lanes, so both the selection
// and the weights are that function's bit for bit.  On return lane j < k
// of wave 0 holds the j-th id and weight (other lanes and waves:
// unspecified).  cand: 64 keys and lgt: kMaxRouteExperts floats of LDS.
__device__ __forceinline__ void block_topk8(const LogitSrc &src, int64_t t, int E, int k,
                                            int renormalize, uint64_t *cand, float *lgt,
                                            int &id, float &wgt) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int nw = (int)(blockDim.x >> 6) < kMaxRouteExperts / 64 ? (int)(blockDim.x >> 6)
                                                                  : kMaxRouteExperts / 64;
  if (wave < nw) {
    const int e = 64 * wave + lane;
    float v[1];
    load_logits(src, t, E, e, v);   // (the element at e, and its store to src.out)
    lgt[e] = v[0];
    const uint64_t key = wave_top8_lanes(e < E ? topk_key(v[0], e) : 0ull, lane);
    if (lane < 8) cand[8 * wave + lane] = key;
  }
  __syncthreads();
  id = 0;
  wgt = 0.0f;
  if (wave == 0) {
    const uint64_t mine = wave_top8_lanes(lane < 8 * nw ? cand[lane] : 0ull, lane);   // lane j: the j-th key
    id = (int)~(uint32_t)mine;
    const uint32_t m = (uint32_t)(mine >> 32);
    const float my_val = __uint_as_float((m & 0x80000000u) ? (m & 0x7FFFFFFFu) : ~m);
    const float lmax =
        __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_val), 0));
    const float ex = lane < k ? expf(my_val - lmax) : 0.0f;
    float denom;
    if (renormalize) {
      denom = wave_sum(ex);
    } else {   // this lane's logits lane + 64 i in i order, as wave_topk_merge adds them
      float sm = 0.0f;
#pragma unroll
      for (int i = 0; i < kMaxRouteExperts / 64; ++i)
        if (lane + 64 * i < E) sm += expf(lgt[lane + 64 * i] - lmax);
      denom = wave_sum(sm);
    }
    wgt = ex / denom;
  }
}

// Permutation by bit-sliced matching: pair p = lane + 64 s sits in slot s of
// its lane (pairs past P carry expert E, above every real one).  Ten ballots
// per slot hold the bits of every pair's expert; walking them from the top
// bit, a lane derives the masks of pairs whose expert equals its own and of
// those whose expert is smaller.  Pair p then goes to
//   (pairs with a smaller expert) + (pairs with the same expert before p),
// which is the stable counting-sort position, and the first pair of each
// expert knows that expert's offset; the offsets of experts without pairs
// are the next larger expert's (a suffix minimum over the experts).
constexpr int kRouteBits = 10;   // expert ids and the sentinel E <= 512

__device__ __forceinline__ int wave_incl_min(int x) {
  constexpr int kMax = 0x7fffffff;
  x = min(x, __builtin_amdgcn_update_dpp(kMax, x, 0x111, 0xF, 0xF, false));   // row_shr:1
  x = min(x, __builtin_amdgcn_update_dpp(kMax, x, 0x112, 0xF, 0xF, false));   // row_shr:2
  x = min(x, __builtin_amdgcn_update_dpp(kMax, x, 0x114, 0xF, 0xF, false));   // row_shr:4
  x = min(x, __builtin_amdgcn_update_dpp(kMax, x, 0x118, 0xF, 0xF, false));   // row_shr:8
  x = min(x, __builtin_amdgcn_update_dpp(kMax, x, 0x142, 0xA, 0xF, false));   // row_bcast:15
  x = min(x, __builtin_amdgcn_update_dpp(kMax, x, 0x143, 0xC, 0xF, false));   // row_bcast:31
  return x;
}

// The stable counting sort of P <= kSmallPairs pairs over E <= 512 experts
// by one wavefront (the workgroup is that one wave: its barriers order the
// LDS array `first`, kMaxRouteExperts entries).  id_of(p) gives pair p's
// expert, an id in 0..E-1.
// With active false a wave only takes part in the barriers (the other waves
// of a larger workgroup).
template <class IdOf>
__device__ void wave_permute_small(IdOf id_of, int P, int E, int32_t *offsets,
                                   int32_t *sorted_pairs, int32_t *first, bool active = true) {
  constexpr int kSlots = kSmallPairs / 64;
  const int lane = threadIdx.x & 63;
  if (!active) {
    __syncthreads();
    __syncthreads();
    return;
  }
  const int nslot = (P + 63) / 64;   // uniform, <= kSlots
  int ev[kSlots];
  uint64_t bits[kSlots][kRouteBits];
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
    const int p = lane + 64 * s;
    ev[s] = p < P ? id_of(p) : E;
#pragma unroll
    for (int b = 0; b < kRouteBits; ++b) bits[s][b] = __builtin_amdgcn_ballot_w64((ev[s] >> b) & 1);
  }
#pragma unroll
  for (int i = 0; i < kMaxRouteExperts / 64; ++i) first[lane + 64 * i] = P;
  __syncthreads();
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
    if (s >= nslot) break;   // uniform
    const int e = ev[s];
    int less = 0, before = 0;
#pragma unroll
    for (int s2 = 0; s2 < kSlots; ++s2) {
      if (s2 >= nslot) break;   // uniform
      uint64_t eq = ~0ull, lt = 0ull;
#pragma unroll
      for (int b = kRouteBits - 1; b >= 0; --b) {
        const uint64_t m = bits[s2][b];
        const bool one = (e >> b) & 1;
        lt = one ? (lt | (eq & ~m)) : lt;
        eq = one ? (eq & m) : (eq & ~m);
      }
      less += __builtin_popcountll(lt);
      if (s2 < s)
        before += __builtin_popcountll(eq);
      else if (s2 == s)
        before += __builtin_amdgcn_mbcnt_hi((uint32_t)(eq >> 32),
                                            __builtin_amdgcn_mbcnt_lo((uint32_t)eq, 0u));
    }
    const int p = lane + 64 * s;
    if (p < P) {
      sorted_pairs[less + before] = p;
      if (before == 0) first[e] = less;   // one writer per expert
    }
  }
  __syncthreads();
  // lane l holds experts 8 (63 - l) .. + 7, so an inclusive min scan over the
  // lanes is a suffix minimum over the experts
  int v[8], lmin = P;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = first[8 * (63 - lane) + i];
    lmin = min(lmin, v[i]);
  }
  const int incl = wave_incl_min(lmin);
  int run = __shfl_up(incl, 1);   // minimum over the larger experts
  if (lane == 0) run = P;
#pragma unroll
  for (int i = 7; i >= 0; --i) {
    run = min(run, v[i]);
    const int e = 8 * (63 - lane) + i;
    if (e < E) offsets[e] = run;
  }
  if (lane == 0) offsets[E] = P;
}

}  // namespace
}  // namespace nvfp4

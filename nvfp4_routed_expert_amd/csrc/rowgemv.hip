// Row-streaming expert-grouped NVFP4 GEMV for decode (W4A16) on gfx950.
//
// Decode cost is the stream of routed-expert weights: each selected expert's
// gate, up and down matrices are read once for the one to few tokens routed
// to it (Eider page, "Performance": prefill batches tokens precisely so
// routed expert weights are reused, which decode cannot do).  This kernel is
// shaped for that stream rather than for a matrix unit:
//
//  * a wavefront reads whole weight rows: for K >= 2048 each of its 64 lanes
//    takes 16 code bytes (32 elements) of a 2048-wide slice, so every load
//    instruction moves one contiguous KiB; for K = 1024 / 512 / 256 a load
//    covers 2 / 4 / 8 rows.  Workgroups of KS = ceil(K / 2048) waves split
//    longer rows and add their partial sums in LDS in a fixed wave order.
//  * each lane's activation slice (the same K positions for every row of the
//    item) is loaded once per item and stays in registers, in bf16 as given;
//  * codes become exact bf16 pairs (v_cvt_scalef32_pk_bf16_fp4, unit scale),
//    multiply the activations in v_dot2_f32_bf16, and each 16-element block
//    sum is scaled once by its E4M3 scale (v_cvt_scalef32_pk_f32_fp8);
//  * eight load steps are kept in flight (a branch-free steady state, so the
//    waits count outstanding loads exactly), and the eight steps' partial
//    sums are reduced across lanes together by one butterfly built from
//    gfx950's v_permlane32_swap / v_permlane16_swap and DPP row moves.
// The butterfly's order is fixed, so results are deterministic.
//
// Each tile row (one token of one expert) is its own work item per block of
// output rows, so an expert with several tokens streams its rows once per
// token; the repeats are close in time and mostly hit L2.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "topk.h"

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

namespace nvfp4 {
namespace {

constexpr int kSlice = 2048;   // K elements covered by one wave (64 lanes x 32)
constexpr int kBatch = 8;      // load steps in flight and reduced together
constexpr int kMaxSlots = 32;  // top-k slots a token-major down item sums
constexpr int kMaxKs = 16;     // K slices (waves) of one unit: K <= 16 * 2048

// ---------------------------------------------------------------------------
// arithmetic
// ---------------------------------------------------------------------------

// 32 codes of one lane -> 16 exact bf16 pairs
__device__ __forceinline__ void decode32(const u32x4 codes, uint32_t (&w)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    w[4 * q + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes[q], 1.0f, 0));
    w[4 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes[q], 1.0f, 1));
    w[4 * q + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes[q], 1.0f, 2));
    w[4 * q + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes[q], 1.0f, 3));
  }
}

// sum over two 16-element blocks, each block sum scaled once by its scale
__device__ __forceinline__ float dot32(const uint32_t (&w)[16], const uint32_t (&a)[16], float s0,
                                       float s1) {
  float b0 = 0.0f, b1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    b0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[i]),
                                         __builtin_bit_cast(bf16x2_t, a[i]), b0, false);
#pragma unroll
  for (int i = 8; i < 16; ++i)
    b1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[i]),
                                         __builtin_bit_cast(bf16x2_t, a[i]), b1, false);
  return b0 * s0 + b1 * s1;
}

// ---------------------------------------------------------------------------
// cross-lane butterfly over 8 values per lane
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}
__device__ __forceinline__ void swap32(float &a, float &b) {   // a=[a_lo,b_lo], b=[a_hi,b_hi]
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a),
                                                  __builtin_bit_cast(uint32_t, b), false, false);
  a = __builtin_bit_cast(float, (uint32_t)r[0]);
  b = __builtin_bit_cast(float, (uint32_t)r[1]);
}
__device__ __forceinline__ void swap16(float &a, float &b) {   // odd 16-rows of a <-> even of b
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, a),
                                                  __builtin_bit_cast(uint32_t, b), false, false);
  a = __builtin_bit_cast(float, (uint32_t)r[0]);
  b = __builtin_bit_cast(float, (uint32_t)r[1]);
}
// One level of the butterfly at lane distance 8, 4 or 2 (the partner differs
// in that lane bit): lanes with the bit set keep index hi, the others lo.
template <int CTRL, int BIT>
__device__ __forceinline__ float pair_level(float lo, float hi, int lane) {
  const bool up = (lane >> BIT) & 1;
  return (up ? hi : lo) + dpp_f32<CTRL>(up ? lo : hi);
}

// v[0..7]: per-lane partial sums of 8 values.  Returns, in every lane, the
// total over the lane's aligned group of G lanes of value idx(lane):
//   G = 64: idx = lane >> 3        G = 32: idx = (lane >> 2) & 7
//   G = 16: idx = (lane >> 1) & 7  G = 8:  idx = lane & 7
template <int G>
__device__ __forceinline__ float reduce8(float (&v)[8], int lane) {
  // 8 -> 4 values
  if constexpr (G == 64) {
#pragma unroll
    for (int j = 0; j < 4; ++j) { swap32(v[j], v[j + 4]); v[j] += v[j + 4]; }
  } else if constexpr (G == 32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) { swap16(v[j], v[j + 4]); v[j] += v[j + 4]; }
  } else if constexpr (G == 16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = pair_level<0x128, 3>(v[j], v[j + 4], lane);   // row_ror:8
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = pair_level<0x141, 2>(v[j], v[j + 4], lane);   // half mirror
  }
  // 4 -> 2 values
  if constexpr (G == 64) {
#pragma unroll
    for (int j = 0; j < 2; ++j) { swap16(v[j], v[j + 2]); v[j] += v[j + 2]; }
  } else if constexpr (G == 32) {
#pragma unroll
    for (int j = 0; j < 2; ++j) v[j] = pair_level<0x128, 3>(v[j], v[j + 2], lane);
  } else if constexpr (G == 16) {
#pragma unroll
    for (int j = 0; j < 2; ++j) v[j] = pair_level<0x141, 2>(v[j], v[j + 2], lane);
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) v[j] = pair_level<0x4E, 1>(v[j], v[j + 2], lane);    // lane ^ 2
  }
  // 2 -> 1 value
  float r;
  if constexpr (G == 64) r = pair_level<0x128, 3>(v[0], v[1], lane);
  else if constexpr (G == 32) r = pair_level<0x141, 2>(v[0], v[1], lane);
  else if constexpr (G == 16) r = pair_level<0x4E, 1>(v[0], v[1], lane);
  else r = pair_level<0xB1, 0>(v[0], v[1], lane);                                     // lane ^ 1
  // plain sums over the lanes still holding the same value
  if constexpr (G == 64) r += dpp_f32<0x141>(r);
  if constexpr (G == 64 || G == 32) r += dpp_f32<0x4E>(r);
  if constexpr (G >= 16) r += dpp_f32<0xB1>(r);
  return r;
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
//
// Work is a flat list of items: item i = (tile row pos = i / groups, group g
// = i % groups of ROWS consecutive output rows).  Tile row pos is the pos-th
// (token, slot) pair in expert order: pair = sorted_pairs[pos], expert =
// topk_ids[pair], token = pair / k (a dense matrix has no routing: pair =
// token = pos, expert 0).  Each unit of KS waves walks items u, u + U, ...
// (U units in the grid) and keeps the next item's weight loads in flight
// while it computes the current one; the routing loads run further ahead
// (pair three items ahead, expert two) so no item waits on a dependent
// chain.  Consecutive units take consecutive row groups, so concurrently
// running waves read neighbouring rows of the same expert, and the tile rows
// of one expert (adjacent positions) share the same XCD, where repeated
// reads of its rows hit L2.

template <int LPR, Epi EPI>
struct RowCfg {
  static constexpr int NMAT = EPI == Epi::SWIGLU ? 2 : 1;
  static constexpr int RPL = 64 / LPR;             // weight rows per load step
  static constexpr int G = LPR;                    // lanes reduced together
  static constexpr int DUP = LPR / kBatch;         // lanes holding the same result
  static constexpr int ROWS = kBatch * RPL;        // output rows per item
};

struct Routing {
  const int32_t *sorted_pairs;   // null: dense
  const int32_t *ids;
  int k;
  bool h_by_pair;                // SWIGLU: write h row `pair` instead of `pos`
};

// WIDE: units of up to 16 waves (K > 4 * 2048) in workgroups of up to 1024
// threads; otherwise at most 4 waves, which leaves the compiler more registers.
template <int LPR, Epi EPI, bool WIDE>
__global__ __launch_bounds__(WIDE ? 1024 : 256) void row_gemv_kernel(const GemmArgs p,
                                                                     const Routing rt, int n_pos) {
  using C = RowCfg<LPR, EPI>;
  constexpr int NMAT = C::NMAT;
  __shared__ float red[((WIDE ? kMaxKs : 4) - 1) * NMAT * 64];   // partial sums of waves 1..

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = p.K, N = p.N;
  const int ks = (K + kSlice - 1) / kSlice;               // waves per unit (K slices)
  const int units_per_wg = (int)(blockDim.x >> 6) / ks;
  const int kw = wave % ks;                               // this wave's K slice
  const int unit = blockIdx.x * units_per_wg + wave / ks;
  const int n_units = gridDim.x * units_per_wg;
  const int sub = lane / LPR, seg = lane % LPR;
  const int kseg = kw * kSlice + 32 * seg;
  const bool kval = kseg < K;
  const uint32_t kc = (uint32_t)min(kseg, K - 32);        // clamped: masked lanes read valid bytes
  const uint32_t code_row = (uint32_t)K / 2, scale_row = (uint32_t)K / 16;
  const int groups = (N + C::ROWS - 1) / C::ROWS;
  const int n_items = n_pos * groups;
  if (unit >= n_items) return;                            // whole unit idle (uniform)

  const uint8_t *cbase[2] = {p.b_codes[0], p.b_codes[NMAT - 1]};
  const uint8_t *sbase[2] = {p.b_scales[0], p.b_scales[NMAT - 1]};
  const float extra = p.extra_scale ? *p.extra_scale : 1.0f;

  // item geometry: byte offsets of this lane's first row
  struct Geo {
    uint32_t code, scale;   // within the expert's matrix
    int64_t ecode, escale;  // expert base offsets
    int e, r0, pos, pair;
  };
  auto geo = [&](int item, int e, int pair) {
    Geo gm;
    gm.pos = item / groups;
    gm.r0 = (item - gm.pos * groups) * C::ROWS;
    gm.e = e;
    gm.pair = pair;
    gm.ecode = (int64_t)e * p.b_codes_estride;
    gm.escale = (int64_t)e * p.b_scales_estride;
    gm.code = (uint32_t)(gm.r0 + sub) * code_row + kc / 2;
    gm.scale = (uint32_t)(gm.r0 + sub) * scale_row + kc / 16;
    return gm;
  };
  const uint32_t last_code = (uint32_t)(N - 1) * code_row + kc / 2;
  const uint32_t last_scale = (uint32_t)(N - 1) * scale_row + kc / 16;
  const uint32_t step_code = (uint32_t)C::RPL * code_row, step_scale = (uint32_t)C::RPL * scale_row;

  u32x4 bq[kBatch][NMAT];
  uint32_t sq[kBatch][NMAT];
  auto load_step = [&](const Geo &gm, int d) {
    const uint32_t oc = min(gm.code + (uint32_t)d * step_code, last_code);
    const uint32_t os = min(gm.scale + (uint32_t)d * step_scale, last_scale);
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      bq[d][m] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4 *>(cbase[m] + gm.ecode + oc));
      sq[d][m] = *reinterpret_cast<const uint16_t *>(sbase[m] + gm.escale + os);
    }
  };
  auto load_a = [&](const Geo &gm, uint32_t (&a)[16]) {
    const int arow = EPI == Epi::SWIGLU ? (gm.pair >= 0 ? gm.pair / rt.k : 0) : gm.pos;
    const uint16_t *src = reinterpret_cast<const uint16_t *>(p.A) + (int64_t)arow * p.lda + kc;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(src + 8 * q);
#pragma unroll
      for (int j = 0; j < 4; ++j) a[4 * q + j] = v[j];
    }
  };
  // later items than the last are clamped to the last (valid, never written)
  auto clamp = [&](int item) { return item < n_items ? item : n_items - 1; };
  auto pair_of = [&](int item) {
    const int pos = clamp(item) / groups;
    return rt.sorted_pairs ? rt.sorted_pairs[pos] : pos;
  };
  // (positions past the kept pairs hold -1: they stream expert 0's rows and
  // write nothing)
  auto expert_of = [&](int pair) { return rt.sorted_pairs && pair >= 0 ? rt.ids[pair] : 0; };

  // prologue: item u loaded; routing of u + U known, pair of u + 2U known
  int item = unit;
  const int pair0 = pair_of(item);
  Geo cur = geo(item, expert_of(pair0), pair0);
  int pair_next = pair_of(item + n_units);
  int e_next = expert_of(pair_next);
  int pair_after = pair_of(item + 2 * n_units);
  uint32_t a_cur[16];
  load_a(cur, a_cur);
#pragma unroll
  for (int d = 0; d < kBatch; ++d) load_step(cur, d);

  for (; item < n_items; item += n_units) {
    // routing two and three items ahead, activations and weights one ahead
    const int e_after = expert_of(pair_after);
    const int pair_after2 = pair_of(item + 3 * n_units);
    const Geo nxt = geo(clamp(item + n_units), e_next, pair_next);
    uint32_t a_nxt[16];
    load_a(nxt, a_nxt);

    float part[NMAT][kBatch];
#pragma unroll
    for (int d = 0; d < kBatch; ++d) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const f32x2_t sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sq[d][m], 1.0f, false);
        uint32_t w[16];
        decode32(bq[d][m], w);
        part[m][d] = kval ? dot32(w, a_cur, sc[0], sc[1]) : 0.0f;
      }
      load_step(nxt, d);
    }
    float r[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) r[m] = reduce8<C::G>(part[m], lane);
    if (ks > 1) {   // partial sums of the K slices, added in wave order
      if (kw > 0) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m) red[((kw - 1) * NMAT + m) * 64 + lane] = r[m];
      }
      __syncthreads();
      if (kw == 0) {
        for (int wv = 1; wv < ks; ++wv) {
#pragma unroll
          for (int m = 0; m < NMAT; ++m) r[m] += red[((wv - 1) * NMAT + m) * 64 + lane];
        }
      }
      __syncthreads();
    }
    // epilogue: the first lane of each duplicate set writes its row
    int idx;
    if constexpr (C::G == 64) idx = lane >> 3;
    else if constexpr (C::G == 32) idx = (lane >> 2) & 7;
    else if constexpr (C::G == 16) idx = (lane >> 1) & 7;
    else idx = lane & 7;
    const int row = cur.r0 + idx * C::RPL + lane / LPR;
    if (kw == 0 && (lane % C::DUP) == 0 && row < N && cur.pair >= 0) {
      if constexpr (EPI == Epi::SWIGLU) {
        const float G = r[0] * p.b_global[0][cur.e] * extra;
        const float U = r[1] * p.b_global[NMAT - 1][cur.e] * extra;
        const uint32_t hb = f32_to_bf16_bits(G / (1.0f + expf(-G)) * U);
        const int64_t hrow = rt.h_by_pair ? cur.pair : cur.pos;
        static_cast<uint16_t *>(p.out)[hrow * p.ldo + row] = (uint16_t)hb;
      } else {
        float v = r[0] * p.b_global[0][cur.e] * extra;
        int64_t orow = cur.pos;
        if constexpr (EPI == Epi::DOWN) {
          orow = cur.pair;
          v *= p.pair_weights[orow];
        }
        if (p.out_type == OutType::F32)
          static_cast<float *>(p.out)[orow * p.ldo + row] = v;
        else
          static_cast<uint16_t *>(p.out)[orow * p.ldo + row] = (uint16_t)f32_to_bf16_bits(v);
      }
    }
    cur = nxt;
    pair_next = pair_after;
    e_next = e_after;
    pair_after = pair_after2;
#pragma unroll
    for (int j = 0; j < 16; ++j) a_cur[j] = a_nxt[j];
  }
}

// Token-major down projection with the combine folded in (decode).  A
// workgroup owns (token t, ROWS consecutive output rows); wave w takes the
// token's slots j = w, w + 4, ... and streams the rows of expert ids[t k + j]
// against h of pair t k + j (h is pair-major), scaled by the expert's global
// and the routing weight.  Wave 0 then adds the slots in order j = 0 .. k-1,
// the same fp32 sum the separate combine would form, and writes y[t].  Only
// for K <= 2048 (one wave per row slice).
template <int LPR>
__global__ __launch_bounds__(256) void row_down_sum_kernel(const GemmArgs p, const int32_t *ids,
                                                           int k) {
  using C = RowCfg<LPR, Epi::DOWN>;
  __shared__ float slot_val[kMaxSlots * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = p.K, N = p.N;
  const int sub = lane / LPR, seg = lane % LPR;
  const int kseg = 32 * seg;
  const bool kval = kseg < K;
  const uint32_t kc = (uint32_t)min(kseg, K - 32);
  const uint32_t code_row = (uint32_t)K / 2, scale_row = (uint32_t)K / 16;
  const int groups = (N + C::ROWS - 1) / C::ROWS;
  const int t = blockIdx.x / groups;
  const int r0 = (blockIdx.x - t * groups) * C::ROWS;
  const float extra = p.extra_scale ? *p.extra_scale : 1.0f;

  // the token's experts and routing weights, lane j holding slot j; a
  // dropped slot (id outside 0..E-1) reads expert 0 and contributes zero
  const int raw_e = lane < k ? ids[t * k + lane] : 0;
  const bool my_keep = (unsigned)raw_e < (unsigned)p.n_experts;
  const int my_e = my_keep ? raw_e : 0;
  const float my_w = lane < k ? p.pair_weights[t * k + lane] : 0.0f;
  const uint64_t keep_mask = __builtin_amdgcn_ballot_w64(my_keep);

  const uint32_t last_code = (uint32_t)(N - 1) * code_row + kc / 2;
  const uint32_t last_scale = (uint32_t)(N - 1) * scale_row + kc / 16;
  const uint32_t step_code = (uint32_t)C::RPL * code_row, step_scale = (uint32_t)C::RPL * scale_row;
  const uint32_t code0 = (uint32_t)(r0 + sub) * code_row + kc / 2;
  const uint32_t scale0 = (uint32_t)(r0 + sub) * scale_row + kc / 16;

  u32x4 bq[kBatch];
  uint32_t sq[kBatch];
  uint32_t a[16];
  auto load = [&](int j) {
    const int e = __builtin_amdgcn_readlane(my_e, j);
    const uint8_t *cb = p.b_codes[0] + (int64_t)e * p.b_codes_estride;
    const uint8_t *sb = p.b_scales[0] + (int64_t)e * p.b_scales_estride;
#pragma unroll
    for (int d = 0; d < kBatch; ++d) {
      const uint32_t oc = min(code0 + (uint32_t)d * step_code, last_code);
      const uint32_t os = min(scale0 + (uint32_t)d * step_scale, last_scale);
      bq[d] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(cb + oc));
      sq[d] = *reinterpret_cast<const uint16_t *>(sb + os);
    }
    const uint16_t *src =
        reinterpret_cast<const uint16_t *>(p.A) + (int64_t)(t * k + j) * p.lda + kc;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(src + 8 * q);
#pragma unroll
      for (int i = 0; i < 4; ++i) a[4 * q + i] = v[i];
    }
  };

  for (int j = wave; j < k; j += 4) {
    load(j);
    float part[kBatch];
#pragma unroll
    for (int d = 0; d < kBatch; ++d) {
      const f32x2_t sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sq[d], 1.0f, false);
      uint32_t w[16];
      decode32(bq[d], w);
      part[d] = kval ? dot32(w, a, sc[0], sc[1]) : 0.0f;
    }
    const float r = reduce8<C::G>(part, lane);
    const int e = __builtin_amdgcn_readlane(my_e, j);
    const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), j));
    slot_val[j * 64 + lane] = r * p.b_global[0][e] * extra * wj;
  }
  __syncthreads();
  if (wave == 0) {
    // kept slots in order j = 0 .. k-1 (the first kept one starts the sum)
    float acc = 0.0f;
    bool any = false;
    for (int j = 0; j < k; ++j) {
      if (!((keep_mask >> j) & 1ull)) continue;   // uniform
      acc = any ? acc + slot_val[j * 64 + lane] : slot_val[j * 64 + lane];
      any = true;
    }
    int idx;
    if constexpr (C::G == 64) idx = lane >> 3;
    else if constexpr (C::G == 32) idx = (lane >> 2) & 7;
    else if constexpr (C::G == 16) idx = (lane >> 1) & 7;
    else idx = lane & 7;
    const int row = r0 + idx * C::RPL + lane / LPR;
    if ((lane % C::DUP) == 0 && row < N) {
      if (p.out_type == OutType::F32)
        static_cast<float *>(p.out)[(int64_t)t * p.ldo + row] = acc;
      else
        static_cast<uint16_t *>(p.out)[(int64_t)t * p.ldo + row] = (uint16_t)f32_to_bf16_bits(acc);
    }
  }
}

template <int LPR, bool WIDE>
hipError_t launch_cfg_w(Epi epi, const GemmArgs &a, const Routing &info, int n_pos, dim3 grid,
                        dim3 block, hipStream_t s) {
  switch (epi) {
    case Epi::LINEAR:
      launch_kernel((row_gemv_kernel<LPR, Epi::LINEAR, WIDE>), grid, block, 0, s, a, info, n_pos);
      break;
    case Epi::SWIGLU:
      launch_kernel((row_gemv_kernel<LPR, Epi::SWIGLU, WIDE>), grid, block, 0, s, a, info, n_pos);
      break;
    case Epi::DOWN:
      launch_kernel((row_gemv_kernel<LPR, Epi::DOWN, WIDE>), grid, block, 0, s, a, info, n_pos);
      break;
  }
  return hipGetLastError();
}

template <int LPR>
hipError_t launch_cfg(Epi epi, const GemmArgs &a, const Routing &info, int n_pos, hipStream_t s) {
  const int ks = (a.K + kSlice - 1) / kSlice;
  const int units_per_wg = ks == 1 ? 4 : 1;
  constexpr int rows = kBatch * (64 / LPR);
  const int64_t groups = (a.N + rows - 1) / rows;
  const int64_t items = groups * (int64_t)n_pos;
  // persistent units: enough to fill every SIMD a few times, never more than items
  int64_t units = 2048 / ks;
  if (units > items) units = items;
  const int64_t blocks = (units + units_per_wg - 1) / units_per_wg;
  const dim3 grid((unsigned)(blocks < 1 ? 1 : blocks)), block(64 * ks * units_per_wg);
  if constexpr (LPR == 64) {
    if (ks > 4) return launch_cfg_w<LPR, true>(epi, a, info, n_pos, grid, block, s);
  }
  return launch_cfg_w<LPR, false>(epi, a, info, n_pos, grid, block, s);
}

template <int LPR>
hipError_t launch_down_sum(const GemmArgs &a, const int32_t *ids, int k, int T, hipStream_t s) {
  constexpr int rows = kBatch * (64 / LPR);
  const int64_t groups = (a.N + rows - 1) / rows;
  const dim3 grid((unsigned)(groups * T)), block(256);
  launch_kernel((row_down_sum_kernel<LPR>), grid, block, 0, s, a, ids, k);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused decode FFN: both projections in one launch (H = 2048)
// ---------------------------------------------------------------------------
//
// One workgroup of kFfnWaves = 16 waves per (tile row pos, slice c of
// kFfnCols = 256 columns of I): the slice's gate and up rows (16 + 16 per
// wave, whole 2048-wide rows per load step as in row_gemv_kernel) give the
// slice of h, bf16-rounded into LDS; the down rows' matching kFfnCols
// columns (8 lanes per row, 8 rows per load step, 128 rows per wave) are
// loaded before the barrier that publishes h, and their dot products with
// the h slice give a partial output row per (pair, slice), scaled by the
// down global and the routing weight.
// ffn_combine_kernel adds the slices and the token's slots in a fixed order.
// One launch streams all three matrices, so the down stream does not pay a
// launch's ramp of its own.
constexpr int kFfnCols = 256;
constexpr int kFfnWaves = 16;
constexpr int kFfnGuRows = kFfnCols / kFfnWaves;        // gate (and up) rows per wave
constexpr int kFfnGuIts = kFfnGuRows / kBatch;           // ... in batches of kBatch
constexpr int kFfnDnRows = 2048 / kFfnWaves;             // down rows per wave (H = 2048)
constexpr int kFfnDnBatches = kFfnDnRows / (8 * kBatch); // 8 rows per load step
static_assert(kFfnGuIts >= 1 && kFfnDnBatches >= 1, "fused FFN split");
constexpr int kXcds = 8;   // consecutive workgroups land on different XCDs

__global__ __launch_bounds__(64 * kFfnWaves) void row_ffn_kernel(const GemmArgs g,
                                                                 const GemmArgs d,
                                                                 const Routing rt,
                                                                 const FfnRoute fr, int n_pos,
                                                                 int n_c, float *ypart) {
  __shared__ uint16_t h_lds[kFfnCols];
  __shared__ int32_t r_ids[kMaxFfnRouteK];
  __shared__ float r_wts[kMaxFfnRouteK];
  __shared__ uint64_t r_cand[kMaxRouteExperts / 8];   // each wave's 8 best keys
  __shared__ float r_logit[kMaxRouteExperts];          // (the full softmax only)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_items = n_pos * n_c;
  const int per = (n_items + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  const int item = (blockIdx.x % kXcds) * per + slot;
  if (slot >= per || item >= n_items) return;   // whole workgroup (uniform)
  const int pos = item / n_c, c = item - pos * n_c;
  // expert order (pair = sorted_pairs[pos]; positions past the kept pairs
  // hold -1), or pair order without a permutation (dropped pairs skipped
  // here by their id), or pair order routed here from the logits
  const int pair = rt.sorted_pairs ? rt.sorted_pairs[pos] : pos;
  if (pair < 0) return;
  const int e_given = fr.logits ? 0 : rt.ids[pair];
  if (!fr.logits && !rt.sorted_pairs && (unsigned)e_given >= (unsigned)g.n_experts) return;
  const int token = pair / rt.k;
  const int H = g.K, I = g.N;   // gate/up: [I, H]; down: [H, I]

  uint32_t a[16];
  {
    const uint16_t *src = reinterpret_cast<const uint16_t *>(g.A) + (int64_t)token * g.lda + 32 * lane;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(src + 8 * q);
#pragma unroll
      for (int j = 0; j < 4; ++j) a[4 * q + j] = v[j];
    }
  }
  // Routed here, while the x row loads are in flight (block_topk8: ids and
  // weights are the routing kernels' bit for bit); the workgroup of slot 0,
  // slice 0 publishes them.
  int e = e_given;
  float route_w = 0.0f;
  if (fr.logits) {   // uniform
    const int j = pair - token * rt.k, k = rt.k;
    int id;
    float wgt;
    block_topk8(LogitSrc{fr.logits, 0, 1, nullptr, nullptr}, token, fr.E, k, fr.renormalize,
                r_cand, r_logit, id, wgt);
    if (wave == 0 && lane < k) {
      r_ids[lane] = id;
      r_wts[lane] = wgt;
      if (j == 0 && c == 0) {
        fr.ids_out[(int64_t)token * k + lane] = id;
        fr.weights_out[(int64_t)token * k + lane] = wgt;
      }
    }
    __syncthreads();
    e = r_ids[j];
    route_w = r_wts[j];
  }

  // ---- gate / up: rows c * kFfnCols + 16 wave + 8 it + step, it = 0..1
  const uint32_t gcode_row = (uint32_t)H / 2, gscale_row = (uint32_t)H / 16;
  const uint8_t *gc[2], *gs[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    gc[m] = g.b_codes[m] + (int64_t)e * g.b_codes_estride + 16 * lane;
    gs[m] = g.b_scales[m] + (int64_t)e * g.b_scales_estride + 2 * lane;
  }
  const int grow0 = c * kFfnCols + kFfnGuRows * wave;
  u32x4 bq[2][kBatch][2];
  uint32_t sq[2][kBatch][2];
  auto load_gu = [&](int buf, int it) {
#pragma unroll
    for (int st = 0; st < kBatch; ++st) {
      const uint32_t row = (uint32_t)(grow0 + 8 * it + st);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        bq[buf][st][m] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(gc[m] + row * gcode_row));
        sq[buf][st][m] = *reinterpret_cast<const uint16_t *>(gs[m] + row * gscale_row);
      }
    }
  };
  const float gg = g.b_global[0][e], gu = g.b_global[1][e];
  load_gu(0, 0);
#pragma unroll
  for (int it = 0; it < kFfnGuIts; ++it) {
    const int cb = it & 1;
    if (it < kFfnGuIts - 1) load_gu(cb ^ 1, it + 1);
    float part[2][kBatch];
#pragma unroll
    for (int st = 0; st < kBatch; ++st) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const f32x2_t sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sq[cb][st][m], 1.0f, false);
        uint32_t w[16];
        decode32(bq[cb][st][m], w);
        part[m][st] = dot32(w, a, sc[0], sc[1]);
      }
    }
    const float G = reduce8<64>(part[0], lane) * gg;
    const float U = reduce8<64>(part[1], lane) * gu;
    if ((lane & 7) == 0)
      h_lds[kFfnGuRows * wave + 8 * it + (lane >> 3)] =
          (uint16_t)f32_to_bf16_bits(G / (1.0f + expf(-G)) * U);
  }

  // ---- down: rows 128 wave + 64 b + 8 st + lane / 8, columns c * kFfnCols +
  // 32 (lane % 8) .. + 32
  const int sub = lane >> 3, seg = lane & 7;
  const uint32_t dcode_row = (uint32_t)I / 2, dscale_row = (uint32_t)I / 16;
  const uint8_t *dc = d.b_codes[0] + (int64_t)e * d.b_codes_estride + c * (kFfnCols / 2) + 16 * seg;
  const uint8_t *ds = d.b_scales[0] + (int64_t)e * d.b_scales_estride + c * (kFfnCols / 16) + 2 * seg;
  const int drow0 = kFfnDnRows * wave + sub;
  u32x4 dq[2][kBatch];
  uint32_t dsq[2][kBatch];
  auto load_d = [&](int buf, int b) {
#pragma unroll
    for (int st = 0; st < kBatch; ++st) {
      const uint32_t row = (uint32_t)(drow0 + 64 * b + 8 * st);
      dq[buf][st] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(dc + row * dcode_row));
      dsq[buf][st] = *reinterpret_cast<const uint16_t *>(ds + row * dscale_row);
    }
  };
  load_d(0, 0);   // independent of h: in flight across the barrier
  __syncthreads();
  uint32_t ah[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
    ah[j] = (uint32_t)h_lds[32 * seg + 2 * j] | ((uint32_t)h_lds[32 * seg + 2 * j + 1] << 16);
  const float scale = d.b_global[0][e] * (fr.logits ? route_w : d.pair_weights[pair]);
  float *yrow = ypart + ((int64_t)pair * n_c + c) * H;
#pragma unroll
  for (int b = 0; b < kFfnDnBatches; ++b) {
    const int cb = b & 1;
    if (b < kFfnDnBatches - 1) load_d(cb ^ 1, b + 1);
    float part[kBatch];
#pragma unroll
    for (int st = 0; st < kBatch; ++st) {
      const f32x2_t sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(dsq[cb][st], 1.0f, false);
      uint32_t w[16];
      decode32(dq[cb][st], w);
      part[st] = dot32(w, ah, sc[0], sc[1]);
    }
    const float r = reduce8<8>(part, lane);
    // lane holds step (lane & 7) of its 8-lane group (row sub = lane / 8)
    yrow[kFfnDnRows * wave + 64 * b + 8 * (lane & 7) + sub] = r * scale;
  }
}

// y[t] = sum over slots j (in order) of sum over slices c (in order) of
// ypart[t k + j][c]: the token's k n_c partial rows are consecutive, so row
// q = j n_c + c; four outputs per thread, sixteen rows' loads in flight (a
// decode step's rows in one round trip), one wave per workgroup so the small
// grid spreads over many CUs.  (Folding this sum into the fused kernel, the
// last workgroup of each token adding the rows, measured slower: the
// store-publish-reload chain it puts at the kernel's end costs more than
// this launch.)
constexpr int kCombineThreads = 64;
constexpr int kCombineBatch = 16;
__global__ __launch_bounds__(kCombineThreads) void ffn_combine_kernel(
    const float *ypart, int64_t T, int64_t H, int k, int n_c, const int32_t *ids, int E, void *y,
    OutType yt, int32_t *offsets, int32_t *sorted_pairs) {
  if (offsets && blockIdx.x == gridDim.x - 1) {   // the extra workgroup: the permutation
    __shared__ int32_t first[kMaxRouteExperts];
    wave_permute_small([&](int p) { return ids[p]; }, (int)T * k, E, offsets, sorted_pairs,
                       first);
    return;
  }
  const int64_t i = ((int64_t)blockIdx.x * kCombineThreads + threadIdx.x) * 4;
  if (i >= T * H) return;
  const int64_t t = i / H, col = i - t * H;
  const int n = k * n_c;
  const float *base = ypart + t * n * H + col;
  // kept slots (ids in 0..E-1) as a bit mask; a dropped slot's rows were
  // never written and are not added
  uint32_t keep = 0;
  for (int j = 0; j < k; ++j) keep |= ((unsigned)ids[t * k + j] < (unsigned)E ? 1u : 0u) << j;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  bool any = false;
  for (int q0 = 0; q0 < n; q0 += kCombineBatch) {
    f32x4 v[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const int q = q0 + u < n ? q0 + u : n - 1;   // (past the end: a valid row, not added)
      v[u] = *reinterpret_cast<const f32x4 *>(base + (int64_t)q * H);
    }
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const int q = q0 + u;
      if (q < n && ((keep >> (q / n_c)) & 1u)) {
        acc = any ? acc + v[u] : v[u];
        any = true;
      }
    }
  }
  if (yt == OutType::F32) {
    *reinterpret_cast<f32x4 *>(static_cast<float *>(y) + i) = acc;
  } else {
    uint16_t *o = static_cast<uint16_t *>(y) + i;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = (uint16_t)f32_to_bf16_bits(acc[q]);
  }
}

// ---------------------------------------------------------------------------
// Dense MLP decode of one row: the gate/up projection over even slices of I
// ---------------------------------------------------------------------------
//
// The decode form of a dense NVFP4 MLP (Eider page, "Qwen3.8 27B": NVFP4 for
// most MLP weights) for a single activation row, where the gate and up rows
// are two thirds of the weight stream.  The rows are dealt out as whole
// 16-column scale blocks of I: with nbt = I / 16 blocks and G = min(nbt,
// kMlpGrid) workgroups, workgroup w takes blocks [w nbt / G, (w + 1) nbt /
// G), at most kMlpMaxNb of them (I = 17408: 1088 blocks, four or five per
// workgroup), so every CU streams the same share (a grid that is not a
// multiple of the CU count would give some CUs two workgroups and double the
// kernel's time; the row GEMV's persistent units do not divide such an I
// evenly either).  Wave v takes the rows c0 + 16 i + v (i < nb) of both
// matrices, whole rows of H per load step with the next row's loads in
// flight, dot products with x held in registers, one cross-lane sum per
// row, and lane 0 writes SiLU * up rounded to bf16.  Sixteen waves per
// workgroup (one workgroup per CU) keep enough loads in flight.  The down
// projection then streams whole rows of K = I (row_mlp_down_kernel below).
// (Carrying each workgroup's h slice on into the matching columns of every
// down row, as the fused routed kernel does, was measured: with slices of
// 64-80 columns each down row gives a workgroup 32-40 bytes, and that
// scattered stream ran at ~1.1 TB/s.)
//
// Lane layout of a row of H = 2048 NP2 + 1024 HALF elements: NP2 pieces of
// 2048 (lane l: elements 32 l .. 32 l + 31 of the piece, 16 code bytes and
// two scale bytes, as in the other row kernels) and, when HALF, one piece of
// 1024 (lane l: 16 elements, 8 code bytes, one scale byte).  x is held in
// registers in the same layout.
constexpr int kMlpWaves = 16;
constexpr int kMlpGrid = 256;    // workgroups: one per CU
constexpr int kMlpMaxNb = 8;     // blocks per workgroup (I <= 16 * 8 * 256)

// 16 codes of one lane -> 8 exact bf16 pairs
__device__ __forceinline__ void decode16(const u32x2 codes, uint32_t (&w)[8]) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    w[4 * q + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes[q], 1.0f, 0));
    w[4 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes[q], 1.0f, 1));
    w[4 * q + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes[q], 1.0f, 2));
    w[4 * q + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes[q], 1.0f, 3));
  }
}

// one 16-element block, its sum scaled once by the block's scale
__device__ __forceinline__ float dot16(const uint32_t (&w)[8], const uint32_t (&a)[8], float s) {
  float b = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    b = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[i]),
                                        __builtin_bit_cast(bf16x2_t, a[i]), b, false);
  return b * s;
}

template <int NP2, bool HALF>
__global__ __launch_bounds__(64 * kMlpWaves, 4) void row_mlp_gate_up_kernel(const GemmArgs g,
                                                                            const int32_t *ids,
                                                                            int nbt, int n_wg) {
  constexpr int H = 2048 * NP2 + (HALF ? 1024 : 0);
  constexpr int NQ = NP2 > 0 ? NP2 : 1;   // (array extents)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int per = (n_wg + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  const int w = (blockIdx.x % kXcds) * per + slot;
  if (slot >= per || w >= n_wg) return;   // whole workgroup (uniform)
  // a dropped token (id outside the experts): no h; the down projection
  // skips it too
  if ((unsigned)ids[0] >= (unsigned)g.n_experts) return;
  const int b0 = (int)((int64_t)w * nbt / n_wg);
  const int nb = (int)((int64_t)(w + 1) * nbt / n_wg) - b0;   // 1 .. kMlpMaxNb (uniform)
  const int c0 = 16 * b0;

  // ---- x row in registers
  uint32_t ax[NQ][16], axh[8];
  {
    const uint16_t *xr = reinterpret_cast<const uint16_t *>(g.A);
#pragma unroll
    for (int q = 0; q < NP2; ++q)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(xr + 2048 * q + 32 * lane + 8 * j);
#pragma unroll
        for (int t = 0; t < 4; ++t) ax[q][4 * j + t] = v[t];
      }
    if constexpr (HALF) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(xr + 2048 * NP2 + 16 * lane + 8 * j);
#pragma unroll
        for (int t = 0; t < 4; ++t) axh[4 * j + t] = v[t];
      }
    }
  }

  // ---- gate / up: rows c0 + 16 i + wave (i < nb) of both matrices
  constexpr uint32_t code_row = H / 2, scale_row = H / 16;
  u32x4 bq[2][2][NQ];   // [buffer][matrix][piece]
  u32x2 bh[2][2];
  uint32_t sq[2][2][NQ], sh[2][2];
  auto load_row = [&](int buf, int i) {
    const uint32_t row = (uint32_t)(c0 + 16 * i + wave);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint8_t *cr = g.b_codes[m] + row * code_row;
      const uint8_t *sr = g.b_scales[m] + row * scale_row;
#pragma unroll
      for (int q = 0; q < NP2; ++q) {
        bq[buf][m][q] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(cr + 1024 * q + 16 * lane));
        sq[buf][m][q] = *reinterpret_cast<const uint16_t *>(sr + 128 * q + 2 * lane);
      }
      if constexpr (HALF) {
        bh[buf][m] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x2 *>(cr + 1024 * NP2 + 8 * lane));
        sh[buf][m] = sr[128 * NP2 + lane];
      }
    }
  };
  // row i from buffer buf: the two sums over the wave (gate in lanes 0..31,
  // up in lanes 32..63 after the first swap), then SiLU * up by lane 0
  auto row_h = [&](int buf, int i) {
    float p[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float acc = 0.0f;
#pragma unroll
      for (int q = 0; q < NP2; ++q) {
        const f32x2_t sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sq[buf][m][q], 1.0f, false);
        uint32_t wd[16];
        decode32(bq[buf][m][q], wd);
        acc += dot32(wd, ax[q], sc[0], sc[1]);
      }
      if constexpr (HALF) {
        const f32x2_t sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sh[buf][m], 1.0f, false);
        uint32_t wd[8];
        decode16(bh[buf][m], wd);
        acc += dot16(wd, axh, sc[0]);
      }
      p[m] = acc;
    }
    swap32(p[0], p[1]);        // p[0] = [gate lo, up lo], p[1] = [gate hi, up hi]
    float r = p[0] + p[1];     // lanes 0..31: gate, 32..63: up (32 partial sums each)
    float r2 = r;
    swap16(r, r2);
    r += r2;
    r += dpp_f32<0x128>(r);    // row_ror:8, 4, 2, 1: every lane of a 16-lane row gets its sum
    r += dpp_f32<0x124>(r);
    r += dpp_f32<0x122>(r);
    r += dpp_f32<0x121>(r);
    const float G = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r), 0)) *
                    g.b_global[0][0];
    const float U = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r), 32)) *
                    g.b_global[1][0];
    if (lane == 0)
      static_cast<uint16_t *>(g.out)[c0 + 16 * i + wave] =
          (uint16_t)f32_to_bf16_bits(G / (1.0f + expf(-G)) * U);
  };
  load_row(0, 0);
  for (int i = 0; i < nb; i += 2) {   // (nb uniform: scalar loop and branches)
    if (i + 1 < nb) load_row(1, i + 1);
    row_h(0, i);
    if (i + 2 < nb) load_row(0, i + 2);
    if (i + 1 < nb) row_h(1, i + 1);
  }

}

// Down projection of the same row: y = g_down w (h . Wd^T), the H output
// rows dealt out evenly over at most kMlpGrid workgroups (H = 5120: 20 rows
// each), so no persistent unit takes an extra row group.  h (I bf16) is
// staged in LDS; a unit is one output row's 2048-wide slice of K (the last
// one shorter), 16 code bytes per lane; wave v takes units v, v + 16, ... in
// batches of eight loads, one butterfly per batch gives the units' sums,
// and thread t adds row t's slices in order and writes y itself (in its
// type; zeros for a dropped token), so no combine launch follows.
constexpr int kMlpDnMaxRows = 32;   // output rows per workgroup
constexpr int kMlpMaxQ = 16;        // 2048-wide slices of K (I <= 32768)

__global__ __launch_bounds__(64 * kMlpWaves, 4) void row_mlp_down_kernel(const GemmArgs d,
                                                                         const int32_t *ids,
                                                                         int n_wg, void *y,
                                                                         OutType yt) {
  extern __shared__ __attribute__((aligned(16))) uint8_t mlp_lds[];
  uint16_t *h_lds = reinterpret_cast<uint16_t *>(mlp_lds);
  const int H = d.N, I = d.K;
  float *sums = reinterpret_cast<float *>(mlp_lds + 2 * (size_t)I);   // [row][slice]
  const int lane = threadIdx.x & 63;
  // (the wave index in a scalar register: the unit bookkeeping below is scalar)
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int per = (n_wg + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  const int w = (blockIdx.x % kXcds) * per + slot;
  if (slot >= per || w >= n_wg) return;   // whole workgroup (uniform)
  const int r0 = (int)((int64_t)w * H / n_wg);
  const int nr = (int)((int64_t)(w + 1) * H / n_wg) - r0;   // 1 .. kMlpDnMaxRows (uniform)
  if ((unsigned)ids[0] >= (unsigned)d.n_experts) {   // a dropped token: zeros
    if ((int)threadIdx.x < nr) {
      if (yt == OutType::F32) static_cast<float *>(y)[r0 + threadIdx.x] = 0.0f;
      else static_cast<uint16_t *>(y)[r0 + threadIdx.x] = 0;
    }
    return;
  }
  // h -> LDS (I is a multiple of 32)
  {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(d.A);
    u32x4 *dst = reinterpret_cast<u32x4 *>(h_lds);
    for (int i = threadIdx.x; i < I / 8; i += 64 * kMlpWaves) dst[i] = src[i];
  }
  const int nq = (I + 2047) / 2048;
  const int nu = nr * nq;
  const uint32_t code_row = (uint32_t)I / 2, scale_row = (uint32_t)I / 16;
  __syncthreads();
  // (one batch in flight per wave: a second, issued before the first is
  // used, measured slower, 14.8 -> 16.8 us at H = 5120, I = 17408)
  const int n_my = (nu - wave + kMlpWaves - 1) / kMlpWaves;   // this wave's units
  for (int b = 0; b * kBatch < n_my; ++b) {   // (scalar loop)
    // the batch's units (wave-uniform): row and slice; a unit past nu, or a
    // lane past the end of K, reads unit 0's first piece (valid, not added)
    int urow[kBatch], uq[kBatch];
    bool ok[kBatch];
#pragma unroll
    for (int st = 0; st < kBatch; ++st) {
      const int u = wave + kMlpWaves * (kBatch * b + st);
      const bool in = u < nu;
      urow[st] = in ? r0 + u / nq : r0;
      uq[st] = in ? u % nq : 0;
      ok[st] = in && 2048 * uq[st] + 32 * lane < I;
    }
    u32x4 cq[kBatch];
    uint32_t sq[kBatch];
#pragma unroll
    for (int st = 0; st < kBatch; ++st) {
      const uint32_t l = ok[st] ? (uint32_t)lane : 0u;
      const uint32_t co = (uint32_t)urow[st] * code_row + 1024u * (uint32_t)uq[st] + 16u * l;
      const uint32_t so = (uint32_t)urow[st] * scale_row + 128u * (uint32_t)uq[st] + 2u * l;
      cq[st] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(d.b_codes[0] + co));
      sq[st] = *reinterpret_cast<const uint16_t *>(d.b_scales[0] + so);
    }
    float part[kBatch];
#pragma unroll
    for (int st = 0; st < kBatch; ++st) {
      uint32_t a[16];
      {
        const u32x4 *hs =
            reinterpret_cast<const u32x4 *>(h_lds + 2048 * uq[st] + 32 * (ok[st] ? lane : 0));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 v = hs[j];
#pragma unroll
          for (int t = 0; t < 4; ++t) a[4 * j + t] = v[t];
        }
      }
      const f32x2_t sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sq[st], 1.0f, false);
      uint32_t wd[16];
      decode32(cq[st], wd);
      const float p = dot32(wd, a, sc[0], sc[1]);
      part[st] = ok[st] ? p : 0.0f;
      // (one unit's h reads at a time: hoisting all eight would spill)
      __builtin_amdgcn_sched_barrier(0);
    }
    const float r = reduce8<64>(part, lane);
    // lane l holds unit 8 b + l / 8 of this wave
    const int u = wave + kMlpWaves * (kBatch * b + (lane >> 3));
    if ((lane & 7) == 0 && u < nu) sums[u] = r;
  }
  __syncthreads();
  if ((int)threadIdx.x >= nr) return;
  float acc = sums[threadIdx.x * nq];
  for (int q = 1; q < nq; ++q) acc += sums[threadIdx.x * nq + q];
  const float v = acc * (d.b_global[0][0] * d.pair_weights[0]);
  if (yt == OutType::F32) static_cast<float *>(y)[r0 + threadIdx.x] = v;
  else static_cast<uint16_t *>(y)[r0 + threadIdx.x] = (uint16_t)f32_to_bf16_bits(v);
}

}  // namespace

bool row_down_sum_supported(int K, int k) {
  return (K == 256 || K == 512 || K == 1024 || K == kSlice) && k >= 1 && k <= kMaxSlots;
}

hipError_t launch_row_down_sum(const GemmArgs &a, const int32_t *ids, int k, int T,
                               hipStream_t s) {
  if (!row_down_sum_supported(a.K, k)) return hipErrorInvalidValue;
  if (a.K == 512) return launch_down_sum<16>(a, ids, k, T, s);
  if (a.K == 256) return launch_down_sum<8>(a, ids, k, T, s);
  if (a.K == 1024) return launch_down_sum<32>(a, ids, k, T, s);
  return launch_down_sum<64>(a, ids, k, T, s);
}

bool row_gemv_supported(int K) {
  if (K % 32 != 0) return false;
  if (K == 256 || K == 512 || K == 1024) return true;
  return K >= kSlice && K <= kMaxKs * kSlice;
}

hipError_t launch_row_gemv(Epi epi, const GemmArgs &a, const int32_t *sorted_pairs,
                           const int32_t *ids, int k, int n_pos, hipStream_t s, bool h_by_pair) {
  const int K = a.K;
  const Routing info{sorted_pairs, ids, k < 1 ? 1 : k, h_by_pair};
  if (K == 512) return launch_cfg<16>(epi, a, info, n_pos, s);    // items of 32 rows
  if (K == 256) return launch_cfg<8>(epi, a, info, n_pos, s);     // items of 64 rows
  if (K == 1024) return launch_cfg<32>(epi, a, info, n_pos, s);   // items of 16 rows
  return launch_cfg<64>(epi, a, info, n_pos, s);                  // items of 8 rows
}

bool row_ffn_supported(int H, int I) { return H == kSlice && I % kFfnCols == 0; }

hipError_t launch_row_ffn(const GemmArgs &g, const GemmArgs &d, const int32_t *sorted_pairs,
                          const int32_t *ids, int k, int P, float *ypart, hipStream_t s,
                          const FfnRoute *route) {
  if (!row_ffn_supported(g.K, g.N) || d.K != g.N || d.N != g.K) return hipErrorInvalidValue;
  FfnRoute fr{};
  if (route) {
    if (sorted_pairs || route->E > kMaxRouteExperts || k > kMaxFfnRouteK) return hipErrorInvalidValue;
    fr = *route;
  }
  const int n_c = g.N / kFfnCols;
  const int64_t items = (int64_t)P * n_c;
  const int64_t grid = (items + kXcds - 1) / kXcds * kXcds;
  const Routing rt{sorted_pairs, ids, k, false};
  launch_kernel(row_ffn_kernel, dim3((unsigned)grid), dim3(64 * kFfnWaves), 0, s, g, d, rt, fr, P,
                n_c, ypart);
  return hipGetLastError();
}

// (H up to 5120: x and two rows' loads stay within the 128 VGPRs of four
// waves per SIMD)
bool row_mlp_supported(int H, int I) {
  return H % 1024 == 0 && H >= 1024 && H <= 5120 && I % 16 == 0 && I >= 16 &&
         (I / 16 + kMlpGrid - 1) / kMlpGrid <= kMlpMaxNb && (int64_t)I * H < ((int64_t)1 << 32);
}

hipError_t launch_row_mlp_gate_up(const GemmArgs &g, const int32_t *ids, hipStream_t s) {
  const int H = g.K, I = g.N;
  if (!row_mlp_supported(H, I)) return hipErrorInvalidValue;
  const int nbt = I / 16, n_wg = nbt < kMlpGrid ? nbt : kMlpGrid;
  const int64_t grid = ((int64_t)n_wg + kXcds - 1) / kXcds * kXcds;
  const dim3 gd((unsigned)grid), bd(64 * kMlpWaves);
#define NVFP4_ROW_MLP(NP2, HALF) \
  launch_kernel((row_mlp_gate_up_kernel<NP2, HALF>), gd, bd, 0, s, g, ids, nbt, n_wg)
  switch (H / 1024) {
    case 1: NVFP4_ROW_MLP(0, true); break;
    case 2: NVFP4_ROW_MLP(1, false); break;
    case 3: NVFP4_ROW_MLP(1, true); break;
    case 4: NVFP4_ROW_MLP(2, false); break;
    case 5: NVFP4_ROW_MLP(2, true); break;
    default: return hipErrorInvalidValue;
  }
#undef NVFP4_ROW_MLP
  return hipGetLastError();
}

// (h and the slice sums within the 64 KB of dynamic LDS a launch gets)
bool row_mlp_down_supported(int H, int I) {
  return I % 32 == 0 && I >= 32 && 2 * (int64_t)I + 4 * kMlpDnMaxRows * kMlpMaxQ <= 65536 && H >= 1 &&
         (H + kMlpGrid - 1) / kMlpGrid <= kMlpDnMaxRows && (int64_t)I * H < ((int64_t)1 << 32);
}

hipError_t launch_row_mlp_down(const GemmArgs &d, const int32_t *ids, void *y, OutType yt,
                               hipStream_t s) {
  const int H = d.N, I = d.K;
  if (!row_mlp_down_supported(H, I)) return hipErrorInvalidValue;
  const int n_wg = H < kMlpGrid ? H : kMlpGrid;
  const int64_t grid = ((int64_t)n_wg + kXcds - 1) / kXcds * kXcds;
  const size_t shm = 2 * (size_t)I + sizeof(float) * kMlpDnMaxRows * kMlpMaxQ;
  launch_kernel(row_mlp_down_kernel, dim3((unsigned)grid), dim3(64 * kMlpWaves), (uint32_t)shm, s,
                d, ids, n_wg, y, yt);
  return hipGetLastError();
}

hipError_t launch_ffn_combine(const float *ypart, int T, int H, int I, int k, const int32_t *ids,
                              int E, void *y, OutType yt, hipStream_t s, int32_t *offsets,
                              int32_t *sorted_pairs) {
  if (H % 4 != 0 || k > 32) return hipErrorInvalidValue;
  if (offsets && (!sorted_pairs || (int64_t)T * k > kSmallPairs || E > kMaxRouteExperts))
    return hipErrorInvalidValue;
  const int64_t threads = ((int64_t)T * H + 3) / 4;
  const int64_t blocks = (threads + kCombineThreads - 1) / kCombineThreads + (offsets ? 1 : 0);
  launch_kernel(ffn_combine_kernel, dim3((unsigned)blocks), dim3(kCombineThreads), 0, s, ypart,
                (int64_t)T, (int64_t)H, k, I / kFfnCols, ids, E, y, yt, offsets, sorted_pairs);
  return hipGetLastError();
}

}  // namespace nvfp4

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
//    instruction moves one contiguous KiB; for K = 512 / 1024 / 256 a load
//    covers 4 / 2 / 8 rows.  Workgroups of KS = ceil(K / 2048) waves split
//    longer rows and add their partial sums in LDS in a fixed wave order.
//  * each lane's activation slice (the same K positions for every row of the
//    item) is loaded once per item and stays in registers, in bf16 as given;
//  * codes become exact bf16 pairs (v_cvt_scalef32_pk_bf16_fp4, unit scale),
//    multiply the activations in v_dot2_f32_bf16, and each 16-element block
//    sum is scaled once by its E4M3 scale (v_cvt_scalef32_pk_f32_fp8);
//  * D row steps of loads are kept in flight ahead of the arithmetic.
// Row sums across lanes use a fixed butterfly, so results are deterministic.
//
// Items: (m-block of up to 16 tile rows of one expert, block of output rows).
// Tile rows are processed in groups of TOK; a block with more rows streams
// its weights once per group.
#include "common.h"
#include "kernels.h"

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

namespace nvfp4 {
namespace {

constexpr int kSlice = 2048;   // K elements covered by one wave (64 lanes x 32)

// Dot product of the 8 E2M1 codes in `word` (as exact bf16 pairs) with
// 8 bf16 activations (4 pairs), accumulated into acc.
__device__ __forceinline__ float dot8(uint32_t word, const uint32_t *a, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 0),
                                        __builtin_bit_cast(bf16x2_t, a[0]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 1),
                                        __builtin_bit_cast(bf16x2_t, a[1]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 2),
                                        __builtin_bit_cast(bf16x2_t, a[2]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 3),
                                        __builtin_bit_cast(bf16x2_t, a[3]), acc, false);
  return acc;
}

// 32 codes (two 16-element blocks with decoded scales s0, s1) against 32
// bf16 activations: each block sum is formed first, then scaled once.
__device__ __forceinline__ float dot32(const u32x4 codes, const uint32_t (&a)[16], float s0,
                                       float s1) {
  const float b0 = dot8(codes[1], a + 4, dot8(codes[0], a + 0, 0.0f));
  const float b1 = dot8(codes[3], a + 12, dot8(codes[2], a + 8, 0.0f));
  return b0 * s0 + b1 * s1;
}

// Sum over each row of 16 lanes (or 8 when LPR == 8) with DPP moves; every
// lane of the row ends with the row's sum.  Fixed order: deterministic.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}

template <int LPR>
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);                          // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_f32<0x4E>(v);                          // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp_f32<0x141>(v);                         // row_half_mirror: the other quad of 8
  if constexpr (LPR >= 16) v += dpp_f32<0x140>(v);   // row_mirror: the other 8 of 16
  return v;
}

__device__ __forceinline__ float lane_value(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// The full sum of weight row u (0 <= u < 64/LPR) of a load step, wave-uniform:
// per-16-lane sums combined in lane order.
template <int LPR>
__device__ __forceinline__ float row_total(float v16, int u) {
  if constexpr (LPR == 64) {
    return (lane_value(v16, 0) + lane_value(v16, 16)) + (lane_value(v16, 32) + lane_value(v16, 48));
  } else if constexpr (LPR == 32) {
    return lane_value(v16, 32 * u) + lane_value(v16, 32 * u + 16);
  } else {
    return lane_value(v16, LPR * u);
  }
}

// LPR: lanes per weight row (64, 32, 16 or 8); TOK: tile rows per pass;
// D: load steps in flight; NMAT: 2 for gate/up (SWIGLU), else 1.
// rows_per_item must be a multiple of D * (64 / LPR) and at most 64.
template <int LPR, int TOK, int D, Epi EPI>
__global__ __launch_bounds__(256) void row_gemv_kernel(const GemmArgs p, int rows_per_item) {
  constexpr int NMAT = EPI == Epi::SWIGLU ? 2 : 1;
  constexpr int RPL = 64 / LPR;                     // rows per load instruction
  __shared__ float red[3][NMAT * TOK * 64];         // partial row sums of waves 1..3

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, ks = blockDim.x >> 6;
  const int K = p.K, N = p.N;
  const int sub = lane / LPR, seg = lane % LPR;     // row within a step, 32-element segment
  const int kseg = wave * kSlice + 32 * seg;        // first K element of this lane
  const bool kval = kseg < K;
  const uint32_t code_row = (uint32_t)K / 2, scale_row = (uint32_t)K / 16;
  const uint32_t kc = (uint32_t)min(kseg, K - 32);  // clamped: masked lanes read valid bytes
  const int row_blocks = (N + rows_per_item - 1) / rows_per_item;
  const int n_mb = p.n_mblocks_dev ? *p.n_mblocks_dev : p.n_mblocks;
  const int n_items = n_mb * row_blocks;
  const int steps = rows_per_item / RPL;            // a multiple of D

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int mb = item / row_blocks, rb = item - mb * row_blocks;
    int e = 0, pos0, nrows;
    if (p.mblocks) {
      const int4 blk = p.mblocks[mb];
      e = blk.x;
      pos0 = blk.y;
      nrows = blk.z;
    } else {
      pos0 = mb * 16;
      nrows = (int)(p.dense_rows - pos0 < 16 ? p.dense_rows - pos0 : 16);
    }
    const int r0 = rb * rows_per_item;
    const uint8_t *cbase[2], *sbase[2];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      cbase[m] = p.b_codes[m] + (int64_t)e * p.b_codes_estride;
      sbase[m] = p.b_scales[m] + (int64_t)e * p.b_scales_estride;
    }
    float gsc[2];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) gsc[m] = p.b_global[m][e];
    const float extra = p.extra_scale ? *p.extra_scale : 1.0f;
    // per-lane byte offsets of this lane's first row (steps add RPL rows)
    const uint32_t lane_code = (uint32_t)(r0 + sub) * code_row + kc / 2;
    const uint32_t lane_scale = (uint32_t)(r0 + sub) * scale_row + kc / 16;
    const uint32_t last_code = (uint32_t)(N - 1) * code_row + kc / 2;
    const uint32_t last_scale = (uint32_t)(N - 1) * scale_row + kc / 16;

    for (int t0 = 0; t0 < nrows; t0 += TOK) {
      // ---- activation slices of this group's tile rows (bf16, zero if absent)
      uint32_t a[TOK][16];
#pragma unroll
      for (int t = 0; t < TOK; ++t) {
        const bool tv = t0 + t < nrows;
        const int arow = tv ? (p.a_rowmap ? p.a_rowmap[pos0 + t0 + t] / p.a_rowdiv : pos0 + t0 + t) : 0;
        const uint16_t *src = reinterpret_cast<const uint16_t *>(p.A) + (int64_t)arow * p.lda + kc;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          u32x4 v = u32x4{0u, 0u, 0u, 0u};
          if (tv && kval) v = *reinterpret_cast<const u32x4 *>(src + 8 * q);
#pragma unroll
          for (int j = 0; j < 4; ++j) a[t][4 * q + j] = v[j];
        }
      }

      // ---- stream the load steps with D of them in flight (branch-free
      //      steady state, so the waits count outstanding loads exactly)
      u32x4 bq[D][NMAT];
      uint32_t sq[D][NMAT];
      float outv[NMAT][TOK];          // lane (row - r0) keeps that row's result
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int t = 0; t < TOK; ++t) outv[m][t] = 0.0f;

#define NVFP4_ROW_LOAD(d, step)                                                           \
      do {                                                                                \
        const uint32_t oc_ = min(lane_code + (uint32_t)(step) * RPL * code_row, last_code);   \
        const uint32_t os_ = min(lane_scale + (uint32_t)(step) * RPL * scale_row, last_scale); \
        _Pragma("unroll") for (int m = 0; m < NMAT; ++m) {                                \
          bq[d][m] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(cbase[m] + oc_)); \
          sq[d][m] = *reinterpret_cast<const uint16_t *>(sbase[m] + os_);                 \
        }                                                                                 \
      } while (0)

#define NVFP4_ROW_STEP(d, step)                                                           \
      do {                                                                                \
        float part_[NMAT][TOK];                                                           \
        _Pragma("unroll") for (int m = 0; m < NMAT; ++m) {                                \
          const f32x2_t sc_ = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sq[d][m], 1.0f, false); \
          _Pragma("unroll") for (int t = 0; t < TOK; ++t)                                 \
            part_[m][t] = row16_sum<LPR>(kval ? dot32(bq[d][m], a[t], sc_[0], sc_[1]) : 0.0f); \
        }                                                                                 \
        _Pragma("unroll") for (int u = 0; u < RPL; ++u) {                                 \
          const int lr_ = (step) * RPL + u;                                               \
          _Pragma("unroll") for (int m = 0; m < NMAT; ++m)                                \
            _Pragma("unroll") for (int t = 0; t < TOK; ++t) {                             \
              const float tot_ = row_total<LPR>(part_[m][t], u);                          \
              outv[m][t] = lane == lr_ ? tot_ : outv[m][t];                               \
            }                                                                             \
        }                                                                                 \
      } while (0)

#pragma unroll
      for (int d = 0; d < D; ++d) NVFP4_ROW_LOAD(d, d);
      int s0 = 0;
      for (; s0 + D < steps; s0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
          NVFP4_ROW_STEP(d, s0 + d);
          NVFP4_ROW_LOAD(d, s0 + d + D);
        }
      }
#pragma unroll
      for (int d = 0; d < D; ++d) NVFP4_ROW_STEP(d, s0 + d);
#undef NVFP4_ROW_LOAD
#undef NVFP4_ROW_STEP

      // ---- the KS waves' partial sums, added in wave order
      if (ks > 1) {
        if (wave > 0) {
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int t = 0; t < TOK; ++t) red[wave - 1][(m * TOK + t) * 64 + lane] = outv[m][t];
        }
        __syncthreads();
        if (wave == 0) {
          for (int w = 1; w < ks; ++w) {
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
              for (int t = 0; t < TOK; ++t) outv[m][t] += red[w - 1][(m * TOK + t) * 64 + lane];
          }
        }
        __syncthreads();
      }

      // ---- epilogue: lane i writes row r0 + i
      const int row = r0 + lane;
      if (wave == 0 && lane < rows_per_item && row < N) {
#pragma unroll
        for (int t = 0; t < TOK; ++t) {
          if (t0 + t >= nrows) break;
          const int pos = pos0 + t0 + t;
          if constexpr (EPI == Epi::SWIGLU) {
            const float G = outv[0][t] * gsc[0] * extra;
            const float U = outv[1][t] * gsc[1] * extra;
            const uint32_t hb = f32_to_bf16_bits(G / (1.0f + expf(-G)) * U);
            static_cast<uint16_t *>(p.out)[(int64_t)pos * p.ldo + row] = (uint16_t)hb;
          } else {
            float v = outv[0][t] * gsc[0] * extra;
            int64_t orow = pos;
            if constexpr (EPI == Epi::DOWN) {
              orow = p.sorted_pairs[pos];
              v *= p.pair_weights[orow];
            }
            if (p.out_type == OutType::F32)
              static_cast<float *>(p.out)[orow * p.ldo + row] = v;
            else
              static_cast<uint16_t *>(p.out)[orow * p.ldo + row] = (uint16_t)f32_to_bf16_bits(v);
          }
        }
      }
    }
  }
}

template <int LPR, int TOK, int D>
hipError_t launch_cfg(Epi epi, const GemmArgs &a, int ks, int rows_per_item, hipStream_t s) {
  const int64_t row_blocks = (a.N + rows_per_item - 1) / rows_per_item;
  int64_t items = row_blocks * (int64_t)a.n_mblocks;
  const int64_t cap = 4096;
  if (items > cap) items = cap;
  if (items < 1) items = 1;
  const dim3 grid((unsigned)items), block(64 * ks);
  switch (epi) {
    case Epi::LINEAR:
      hipLaunchKernelGGL((row_gemv_kernel<LPR, TOK, D, Epi::LINEAR>), grid, block, 0, s, a,
                         rows_per_item);
      break;
    case Epi::SWIGLU:
      hipLaunchKernelGGL((row_gemv_kernel<LPR, TOK, D, Epi::SWIGLU>), grid, block, 0, s, a,
                         rows_per_item);
      break;
    case Epi::DOWN:
      hipLaunchKernelGGL((row_gemv_kernel<LPR, TOK, D, Epi::DOWN>), grid, block, 0, s, a,
                         rows_per_item);
      break;
  }
  return hipGetLastError();
}

}  // namespace

bool row_gemv_supported(int K) {
  if (K % 32 != 0) return false;
  if (K == 256 || K == 512 || K == 1024) return true;
  return K >= kSlice && K <= 4 * kSlice;
}

hipError_t launch_row_gemv(Epi epi, const GemmArgs &a, hipStream_t s) {
  const int K = a.K;
  if (K == 512) return launch_cfg<16, 2, 8>(epi, a, 1, 64, s);    // 16 steps of 4 rows
  if (K == 256) return launch_cfg<8, 2, 4>(epi, a, 1, 64, s);     // 8 steps of 8 rows
  if (K == 1024) return launch_cfg<32, 2, 8>(epi, a, 1, 32, s);   // 16 steps of 2 rows
  const int ks = (K + kSlice - 1) / kSlice;
  return launch_cfg<64, 2, 8>(epi, a, ks, 32, s);                 // 32 steps of 1 row
}

}  // namespace nvfp4

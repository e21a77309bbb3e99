// Small-M expert-grouped NVFP4 GEMV (decode) on gfx950.
//
// In decode a routed expert sees one to a few tokens, so its weights are read
// once and used by a handful of rows: the kernel is an HBM stream, and the
// pages place decode cost in exactly this weight streaming (Eider page,
// "Performance": prefill batches tokens precisely so routed expert weights
// are reused; decode cannot).  On MI355X the loaded HBM latency is several
// microseconds, so the stream only reaches bandwidth with tens of MB in
// flight.  The kernel therefore gives each wave many weight rows (NF
// fragments of 16 rows) of one 128-wide K chunk at a time, so that one
// activation fragment serves NF fragments of weights, and keeps D chunks of
// 128-bit loads outstanding; the KS waves of a workgroup split K and meet in
// LDS in a fixed wave order (deterministic).
//
// MFMA operand layout and K permutation as in the grouped GEMM (gemm.hip):
// lane l holds weight row l%16 of a fragment; lane group g = l/16 covers the
// 32 K-elements 32g..32g+31 of a chunk, 8 per k-step.
//
// bf16 A rows (ABF16): the workgroup computes each row's maximum and converts
// the row to fp16 with the power-of-two shift that makes it exact (as the row
// preparation kernel does) while loading it, so h needs no separate pass.
#include "common.h"
#include "kernels.h"

namespace nvfp4 {
namespace {

constexpr int kChunk = 128;

template <int KS, int NF, int D, Epi EPI, bool ABF16>
__global__ __launch_bounds__(KS * 64) void grouped_gemv_kernel(const GemmArgs p) {
  static_assert(EPI != Epi::SWIGLU || NF % 2 == 0, "gate/up fragments pair up");
  constexpr int kCols = (EPI == Epi::SWIGLU ? NF / 2 : NF) * 16;
  constexpr int kHalf = EPI == Epi::SWIGLU ? NF / 2 : NF;   // fragments per matrix
  __shared__ f32x4 red[KS > 1 ? (KS - 1) * NF * 64 : 1];
  __shared__ int lds_shift[16];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int K = p.K, N = p.N;
  const int n_tiles = (N + kCols - 1) / kCols;
  const int n_mb = p.n_mblocks_dev ? *p.n_mblocks_dev : p.n_mblocks;
  const int n_items = n_mb * n_tiles;
  const float extra = p.extra_scale ? *p.extra_scale : 1.0f;
  const int nchunks = (K + kChunk - 1) / kChunk;
  const int mine = wave < nchunks ? (nchunks - wave + KS - 1) / KS : 0;
  const uint32_t code_row = (uint32_t)K / 2, scale_row = (uint32_t)K / 16;

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int mb = item / n_tiles, nt = item - mb * n_tiles;
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
    const int col0 = nt * kCols;

    // wave-uniform expert bases, per-lane 32-bit row offsets
    const uint8_t *cb0 = p.b_codes[0] + (int64_t)e * p.b_codes_estride;
    const uint8_t *sb0 = p.b_scales[0] + (int64_t)e * p.b_scales_estride;
    const uint8_t *cb1 = cb0, *sb1 = sb0;
    if constexpr (EPI == Epi::SWIGLU) {
      cb1 = p.b_codes[1] + (int64_t)e * p.b_codes_estride;
      sb1 = p.b_scales[1] + (int64_t)e * p.b_scales_estride;
    }
    const int row0 = col0 + lr;   // weight row of fragment 0 (of each matrix)

    const bool aval = lr < nrows;
    int arow = 0;
    if (aval) arow = p.a_rowmap ? p.a_rowmap[pos0 + lr] / p.a_rowdiv : pos0 + lr;
    const char *abase = reinterpret_cast<const char *>(p.A) + (int64_t)arow * p.lda * 2;

    int ash = 0;
    if constexpr (ABF16) {
      for (int r = wave; r < nrows; r += KS) {
        const int ar = p.a_rowmap ? p.a_rowmap[pos0 + r] / p.a_rowdiv : pos0 + r;
        const uint16_t *row = reinterpret_cast<const uint16_t *>(p.A) + (int64_t)ar * p.lda;
        float m = 0.0f;
        for (int c = lane * 8; c < K; c += 512) {
          const u32x4 w = *reinterpret_cast<const u32x4 *>(row + c);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            m = fmaxf(m, fmaxf(__builtin_fabsf(__uint_as_float(w[i] << 16)),
                               __builtin_fabsf(__uint_as_float(w[i] & 0xFFFF0000u))));
        }
        m = wave_max(m);
        if (lane == 0) lds_shift[r] = m > 0.0f ? exponent_of(m) - 15 : 0;
      }
      __syncthreads();
      ash = aval ? lds_shift[lr] : 0;
    }

    // Per-lane 32-bit offsets of each fragment's weight row.  Rows past N and
    // K segments past K are clamped to valid memory: their products only
    // meet zero activations (A is zeroed there) or unused output columns.
    uint32_t boff[NF], soff[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int rr = min(row0 + 16 * (f % kHalf), N - 1);
      boff[f] = (uint32_t)rr * code_row;
      soff[f] = (uint32_t)rr * scale_row;
    }
    const uint8_t *cbase[2] = {cb0, cb1};
    const uint8_t *sbase[2] = {sb0, sb1};

    f32x4 acc[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 bq[D][NF];
    uint32_t sq[D][NF];
    u32x4 aq[D][4];

#define NVFP4_GEMV_LOAD(d, c)                                                            \
    do {                                                                                 \
      const int kk_ = (c) * kChunk + 32 * lg;                                            \
      const uint32_t kc_ = (uint32_t)min(kk_, K - 32);                                   \
      _Pragma("unroll") for (int f = 0; f < NF; ++f) {                                   \
        const int m_ = f < kHalf ? 0 : 1;                                                \
        bq[d][f] = __builtin_nontemporal_load(                                           \
            reinterpret_cast<const u32x4 *>(cbase[m_] + (boff[f] + kc_ / 2)));           \
        sq[d][f] = *reinterpret_cast<const uint16_t *>(sbase[m_] + (soff[f] + kc_ / 16)); \
      }                                                                                  \
      const bool av_ = aval && kk_ < K;                                                  \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                    \
        aq[d][i] = u32x4{0u, 0u, 0u, 0u};                                                \
        if (av_) aq[d][i] = *reinterpret_cast<const u32x4 *>(abase + ((int64_t)kk_ + 8 * i) * 2); \
      }                                                                                  \
    } while (0)

#define NVFP4_GEMV_COMPUTE(d)                                                            \
    do {                                                                                 \
      f16x8 av_[4];                                                                      \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                    \
        if constexpr (ABF16) {                                                           \
          _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                \
            const uint32_t w_ = aq[d][i][q];                                             \
            av_[i][2 * q] = (_Float16)__builtin_ldexpf(__uint_as_float(w_ << 16), -ash); \
            av_[i][2 * q + 1] =                                                          \
                (_Float16)__builtin_ldexpf(__uint_as_float(w_ & 0xFFFF0000u), -ash);     \
          }                                                                              \
        } else {                                                                         \
          av_[i] = __builtin_bit_cast(f16x8, aq[d][i]);                                  \
        }                                                                                \
      }                                                                                  \
      _Pragma("unroll") for (int f = 0; f < NF; ++f) {                                   \
        f16x2 s0_, s1_;                                                                  \
        e4m3x2_to_f16_pairs(sq[d][f], s0_, s1_);                                         \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                  \
          const f16x8 b_ = dequant8_f16(bq[d][f][i], i < 2 ? s0_ : s1_);                 \
          acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av_[i], b_, acc[f], 0, 0, 0);  \
        }                                                                                \
        __builtin_amdgcn_sched_barrier(0);                                               \
      }                                                                                  \
    } while (0)

    // this wave's chunks are wave, wave + KS, ...; D of them in flight
    if (mine > 0) NVFP4_GEMV_LOAD(0, wave);
    if constexpr (D > 1) {
      if (mine > 1) NVFP4_GEMV_LOAD(1, wave + KS);
      for (int i = 0; i < mine; i += 2) {
        NVFP4_GEMV_COMPUTE(0);
        if (i + 2 < mine) NVFP4_GEMV_LOAD(0, wave + KS * (i + 2));
        if (i + 1 < mine) {
          NVFP4_GEMV_COMPUTE(1);
          if (i + 3 < mine) NVFP4_GEMV_LOAD(1, wave + KS * (i + 3));
        }
      }
    } else {
      for (int i = 0; i < mine; ++i) {
        NVFP4_GEMV_COMPUTE(0);
        if (i + 1 < mine) NVFP4_GEMV_LOAD(0, wave + KS * (i + 1));
      }
    }
#undef NVFP4_GEMV_LOAD
#undef NVFP4_GEMV_COMPUTE

    // ---- reduce the KS partial tiles in wave order
    if constexpr (KS > 1) {
      if (wave > 0) {
#pragma unroll
        for (int f = 0; f < NF; ++f) red[((wave - 1) * NF + f) * 64 + lane] = acc[f];
      }
      __syncthreads();
      if (wave == 0) {
        for (int w = 1; w < KS; ++w) {
#pragma unroll
          for (int f = 0; f < NF; ++f) acc[f] += red[((w - 1) * NF + f) * 64 + lane];
        }
      }
    }

    // ---- epilogue (wave 0): lane holds rows 4*lg + j, column lr of each fragment
    if (wave == 0) {
      int sh[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * lg + j;
        sh[j] = 0;
        if (r < nrows) {
          if constexpr (ABF16) {
            sh[j] = lds_shift[r];
          } else if (p.a_shift) {
            const int ar = p.a_rowmap ? p.a_rowmap[pos0 + r] / p.a_rowdiv : pos0 + r;
            sh[j] = p.a_shift[ar];
          }
        }
      }
      if constexpr (EPI == Epi::SWIGLU) {
        float amax = 0.0f;
        const float gg = p.b_global[0][e], gu = p.b_global[1][e];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * lg + j;
          if (r >= nrows) continue;
          uint16_t *hrow = static_cast<uint16_t *>(p.out) + (int64_t)(pos0 + r) * p.ldo;
#pragma unroll
          for (int f = 0; f < kHalf; ++f) {
            const int col = col0 + f * 16 + lr;
            if (col >= N) continue;
            const float G = __builtin_ldexpf(acc[f][j], sh[j]) * gg * extra;
            const float U = __builtin_ldexpf(acc[f + kHalf][j], sh[j]) * gu * extra;
            const uint32_t hb = f32_to_bf16_bits(G / (1.0f + expf(-G)) * U);
            hrow[col] = (uint16_t)hb;
            amax = fmaxf(amax, __builtin_fabsf(bf16_bits_to_f32(hb)));
          }
        }
        if (p.amax_slot) {
          amax = wave_max(amax);
          if (lane == 0 && amax > 0.0f) atomicMax(p.amax_slot, __float_as_uint(amax));
        }
      } else {
        const float gw = p.b_global[0][e];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * lg + j;
          if (r >= nrows) continue;
          const int pos = pos0 + r;
          int64_t orow = pos;
          float w = 1.0f;
          if constexpr (EPI == Epi::DOWN) {
            orow = p.sorted_pairs[pos];
            w = p.pair_weights[orow];
          }
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            const int col = col0 + f * 16 + lr;
            if (col >= N) continue;
            float v = __builtin_ldexpf(acc[f][j], sh[j]) * gw * extra;
            if constexpr (EPI == Epi::DOWN) v *= w;
            if (p.out_type == OutType::F32)
              static_cast<float *>(p.out)[orow * p.ldo + col] = v;
            else
              static_cast<uint16_t *>(p.out)[orow * p.ldo + col] = (uint16_t)f32_to_bf16_bits(v);
          }
        }
      }
    }
    if constexpr (KS > 1 || ABF16) __syncthreads();   // LDS reuse by the next item
  }
}

template <int KS, int NF, int D>
hipError_t launch_cfg(Epi epi, const GemmArgs &a, bool a_bf16, hipStream_t s) {
  const int cols = (epi == Epi::SWIGLU ? NF / 2 : NF) * 16;
  const int64_t n_tiles = (a.N + cols - 1) / cols;
  int64_t items = n_tiles * (int64_t)a.n_mblocks;
  const int64_t cap = 8192 / KS;
  if (items > cap) items = cap;
  if (items < 1) items = 1;
  const dim3 grid((unsigned)items), block(KS * 64);
#define NVFP4_GEMV_CASE(EPIV)                                                               \
  if (a_bf16)                                                                               \
    launch_kernel((grouped_gemv_kernel<KS, NF, D, EPIV, true>), grid, block, 0, s, a);  \
  else                                                                                      \
    launch_kernel((grouped_gemv_kernel<KS, NF, D, EPIV, false>), grid, block, 0, s, a);
  switch (epi) {
    case Epi::LINEAR: NVFP4_GEMV_CASE(Epi::LINEAR) break;
    case Epi::SWIGLU: NVFP4_GEMV_CASE(Epi::SWIGLU) break;
    case Epi::DOWN: NVFP4_GEMV_CASE(Epi::DOWN) break;
  }
#undef NVFP4_GEMV_CASE
  return hipGetLastError();
}

}  // namespace

// Tiles of 8 fragments (128 weight rows; gate/up: 64 h columns).  K is split
// over up to 8 waves; short K uses fewer waves so each keeps a full chunk.
int gemv_tile_cols(Epi epi, int N, int K) {
  (void)N;
  (void)K;
  return epi == Epi::SWIGLU ? 64 : 128;
}

hipError_t launch_gemv(Epi epi, const GemmArgs &a, bool a_bf16, hipStream_t s) {
  const int nchunks = (a.K + kChunk - 1) / kChunk;
  if (nchunks <= 4) return launch_cfg<4, 8, 1>(epi, a, a_bf16, s);
  if (nchunks <= 8) return launch_cfg<8, 8, 1>(epi, a, a_bf16, s);
  return launch_cfg<8, 8, 2>(epi, a, a_bf16, s);
}

}  // namespace nvfp4

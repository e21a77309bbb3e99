// Expert-grouped NVFP4 GEMM on gfx950 MFMA, with the routed-FFN epilogues.
//
// The routed-expert FFN streams each selected expert's weights once per
// batch of tokens that share it: a grouped GEMV in decode and a grouped GEMM
// over prefill chunks of up to 512 tokens (Eider page, "Performance").  One
// kernel covers both: a work item is (expert, block of up to BM tile rows,
// tile of weight rows).  Weights are read straight from HBM with 128-bit
// loads, dequantised in registers (E2M1 -> fp16 by the packed converter,
// times the E4M3 block scale in packed fp16; exact, since every product has
// at most 6 significant bits) and fed to v_mfma_f32_16x16x32_f16.  The
// activations arrive as exact fp16 rows (see the row preparation kernel).
//
// K permutation.  For MFMA 16x16x32 lane l supplies k = 8*(l/16) .. +8 of
// each 32-wide step.  Over a 128-wide chunk the four steps i = 0..3 are
// assigned so that lane group g = l/16 covers k = 32g + 8i .. +8: one 16-byte
// load then gives a lane all 32 codes (and both block scales) it needs for
// the chunk.  A and B use the same assignment, so the dot product is
// unchanged.
#include "common.h"
#include "kernels.h"

namespace nvfp4 {
namespace {

constexpr int kChunk = 128;

template <int NW, int NF, int MS, Epi EPI>
__global__ __launch_bounds__(NW * 64) void grouped_gemm_kernel(const GemmArgs p) {
  static_assert(EPI != Epi::SWIGLU || NF % 2 == 0, "gate/up fragments pair up");
  constexpr int kColsPerWave = (EPI == Epi::SWIGLU ? NF / 2 : NF) * 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int K = p.K, N = p.N;
  const int n_out = N;   // output columns: weight rows (SWIGLU: h columns)
  const int n_tiles = (n_out + NW * kColsPerWave - 1) / (NW * kColsPerWave);
  const int n_mb = p.n_mblocks_dev ? *p.n_mblocks_dev : p.n_mblocks;
  const int n_items = n_mb * n_tiles;
  const float extra = p.extra_scale ? *p.extra_scale : 1.0f;

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int mb = item / n_tiles, nt = item - mb * n_tiles;
    int e = 0, pos0, nrows;
    if (p.mblocks) {
      const int4 blk = p.mblocks[mb];
      e = blk.x;
      pos0 = blk.y;
      nrows = blk.z;
    } else {   // dense: consecutive blocks of MS*16 rows of one matrix
      pos0 = mb * (MS * 16);
      nrows = (int)(p.dense_rows - pos0 < MS * 16 ? p.dense_rows - pos0 : MS * 16);
    }
    const int col0 = (nt * NW + wave) * kColsPerWave;

    // weight rows of this lane, one per fragment
    const uint8_t *bc[NF];
    const uint8_t *bs[NF];
    bool bval[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int mat = (EPI == Epi::SWIGLU && f >= NF / 2) ? 1 : 0;
      const int fr = (EPI == Epi::SWIGLU) ? (f % (NF / 2)) : f;
      const int row = col0 + fr * 16 + lr;
      bval[f] = row < N;
      const int rr = bval[f] ? row : 0;
      bc[f] = p.b_codes[mat] + (int64_t)e * p.b_codes_estride + (int64_t)rr * (K / 2);
      bs[f] = p.b_scales[mat] + (int64_t)e * p.b_scales_estride + (int64_t)rr * (K / 16);
    }
    // activation rows of this lane, one per 16-row subtile
    const _Float16 *ap[MS];
    bool aval[MS];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      const int r = ms * 16 + lr;
      aval[ms] = r < nrows;
      int arow = 0;
      if (aval[ms]) arow = p.a_rowmap ? p.a_rowmap[pos0 + r] / p.a_rowdiv : pos0 + r;
      ap[ms] = p.A + (int64_t)arow * p.lda;
    }

    f32x4 acc[MS][NF];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[ms][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < K; k0 += kChunk) {
      const int kk = k0 + 32 * lg;
      const bool kv = kk < K;
      u32x4 bw[NF];
      uint32_t bsc[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        if (bval[f] && kv) {
          bw[f] = *reinterpret_cast<const u32x4 *>(bc[f] + kk / 2);
          bsc[f] = *reinterpret_cast<const uint16_t *>(bs[f] + kk / 16);
        } else {
          bw[f] = u32x4{0u, 0u, 0u, 0u};
          bsc[f] = 0u;
        }
      }
      f16x2 sc0[NF], sc1[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f) e4m3x2_to_f16_pairs(bsc[f], sc0[f], sc1[f]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f16x8 bf[NF];
#pragma unroll
        for (int f = 0; f < NF; ++f) bf[f] = dequant8_f16(bw[f][i], i < 2 ? sc0[f] : sc1[f]);
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
          if (ms * 16 >= nrows) break;   // wave-uniform: skip empty subtiles
          f16x8 a = {0, 0, 0, 0, 0, 0, 0, 0};
          if (aval[ms] && kv) a = *reinterpret_cast<const f16x8 *>(ap[ms] + kk + 8 * i);
#pragma unroll
          for (int f = 0; f < NF; ++f)
            acc[ms][f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bf[f], acc[ms][f], 0, 0, 0);
        }
      }
    }

    // ---- epilogue: lane holds rows 4*lg + j (j = 0..3) of each subtile,
    //      column lr of each fragment.
    if constexpr (EPI == Epi::SWIGLU) {
      float amax = 0.0f;
      const float gg = p.b_global[0][e], gu = p.b_global[1][e];
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = ms * 16 + 4 * lg + j;
          if (r >= nrows) continue;
          const int pos = pos0 + r;
          const int arow = p.a_rowmap ? p.a_rowmap[pos] / p.a_rowdiv : pos;
          const int sh = p.a_shift ? p.a_shift[arow] : 0;
          uint16_t *hrow = static_cast<uint16_t *>(p.out) + (int64_t)pos * p.ldo;
#pragma unroll
          for (int f = 0; f < NF / 2; ++f) {
            const int col = col0 + f * 16 + lr;
            if (col >= N) continue;
            const float G = __builtin_ldexpf(acc[ms][f][j], sh) * gg * extra;
            const float U = __builtin_ldexpf(acc[ms][f + NF / 2][j], sh) * gu * extra;
            const float hv = G / (1.0f + expf(-G)) * U;
            const uint32_t hb = f32_to_bf16_bits(hv);
            hrow[col] = (uint16_t)hb;
            amax = fmaxf(amax, __builtin_fabsf(bf16_bits_to_f32(hb)));
          }
        }
      }
      if (p.amax_slot) {
        amax = wave_max(amax);
        if (lane == 0 && amax > 0.0f) atomicMax(p.amax_slot, __float_as_uint(amax));
      }
    } else {
      const float gw = p.b_global[0][e];
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = ms * 16 + 4 * lg + j;
          if (r >= nrows) continue;
          const int pos = pos0 + r;
          const int arow = p.a_rowmap ? p.a_rowmap[pos] / p.a_rowdiv : pos;
          const int sh = p.a_shift ? p.a_shift[arow] : 0;
          int64_t orow = pos;
          float w = 1.0f;
          if constexpr (EPI == Epi::DOWN) {
            const int pair = p.sorted_pairs[pos];
            orow = pair;
            w = p.pair_weights[pair];
          }
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            const int col = col0 + f * 16 + lr;
            if (col >= N) continue;
            float v = __builtin_ldexpf(acc[ms][f][j], sh) * gw * extra;
            if constexpr (EPI == Epi::DOWN) v *= w;
            if (p.out_type == OutType::F32)
              static_cast<float *>(p.out)[orow * p.ldo + col] = v;
            else
              static_cast<uint16_t *>(p.out)[orow * p.ldo + col] = (uint16_t)f32_to_bf16_bits(v);
          }
        }
      }
    }
  }
}

template <int NW, int NF, int MS>
hipError_t launch_cfg(Epi epi, const GemmArgs &a, hipStream_t s) {
  constexpr int cols_lin = NF * 16, cols_swi = NF / 2 * 16;
  const int cols = (epi == Epi::SWIGLU) ? cols_swi : cols_lin;
  const int64_t n_tiles = (a.N + NW * cols - 1) / (NW * cols);
  int64_t items = n_tiles * (int64_t)a.n_mblocks;
  const int64_t cap = 2048 / NW;
  if (items > cap) items = cap;
  if (items < 1) items = 1;
  const dim3 grid((unsigned)items), block(NW * 64);
  switch (epi) {
    case Epi::LINEAR:
      launch_kernel((grouped_gemm_kernel<NW, NF, MS, Epi::LINEAR>), grid, block, 0, s, a);
      break;
    case Epi::SWIGLU:
      launch_kernel((grouped_gemm_kernel<NW, NF, MS, Epi::SWIGLU>), grid, block, 0, s, a);
      break;
    case Epi::DOWN:
      launch_kernel((grouped_gemm_kernel<NW, NF, MS, Epi::DOWN>), grid, block, 0, s, a);
      break;
  }
  return hipGetLastError();
}

// m-blocks of up to bm rows for every expert with pairs, built by one
// workgroup of any size (multiple of 64, at most 1024 threads).
__device__ void build_plan(const int32_t *offsets, int E, int bm, int4 *mblocks,
                           int32_t *n_mblocks) {
  __shared__ int32_t wave_tot[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthreads = blockDim.x, nwaves = nthreads >> 6;
  int run = 0;   // m-blocks of experts handled by earlier passes
  for (int e0 = 0; e0 < E; e0 += nthreads) {
    const int e = e0 + tid;
    int lo = 0, c = 0;
    if (e < E) {
      lo = offsets[e];
      c = offsets[e + 1] - lo;
    }
    const int nb = (c + bm - 1) / bm;
    int incl = nb;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int wbase = run;
    for (int w = 0; w < wave; ++w) wbase += wave_tot[w];
    const int first = wbase + incl - nb;
    for (int b = 0; b < nb; ++b) {
      const int r0 = b * bm;
      mblocks[first + b] = int4{e, lo + r0, (c - r0) < bm ? (c - r0) : bm, 0};
    }
    int total = 0;
    for (int w = 0; w < nwaves; ++w) total += wave_tot[w];
    __syncthreads();
    run += total;
  }
  if (tid == 0) *n_mblocks = run;
}

// A second list of bm2-row blocks (a different block size for the down
// projection) when mblocks2 is set.
__global__ __launch_bounds__(1024) void moe_plan_kernel(const int32_t *offsets, int E, int bm,
                                                        int4 *mblocks, int32_t *n_mblocks,
                                                        int bm2, int4 *mblocks2,
                                                        int32_t *n_mblocks2, uint32_t *zero,
                                                        int zero_words) {
  for (int i = threadIdx.x; i < zero_words; i += blockDim.x) zero[i] = 0u;
  build_plan(offsets, E, bm, mblocks, n_mblocks);
  if (mblocks2) build_plan(offsets, E, bm2, mblocks2, n_mblocks2);
}

// Blocks before the last: x rows -> fp16 with their power-of-two shift (as
// the row preparation kernel's SHIFT mode), one wavefront per row, or for
// few rows (wide) one workgroup per row.  The last block builds the plan and
// zeroes the scratch words.
__global__ __launch_bounds__(256) void moe_prep_kernel(const uint16_t *x, int64_t T, int64_t H,
                                                       _Float16 *x16, int32_t *xshift,
                                                       const int32_t *offsets, int E, int bm,
                                                       int4 *mblocks, int32_t *n_mblocks, int bm2,
                                                       int4 *mblocks2, int32_t *n_mblocks2,
                                                       uint32_t *zero, int64_t zero_words,
                                                       int wide) {
  if (blockIdx.x == gridDim.x - 1) {
    for (int64_t i = threadIdx.x; i < zero_words; i += blockDim.x) zero[i] = 0u;
    build_plan(offsets, E, bm, mblocks, n_mblocks);
    if (mblocks2) build_plan(offsets, E, bm2, mblocks2, n_mblocks2);
    return;
  }
  __shared__ float wmax[4];
  const int lane = threadIdx.x & 63;
  const int64_t r = wide ? (int64_t)blockIdx.x : (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= T) return;
  const int t0 = wide ? threadIdx.x : lane;
  const int step = wide ? 256 * 8 : 512;
  const uint16_t *row = x + r * H;
  float m = 0.0f;
  for (int64_t c = t0 * 8; c < H; c += step) {
    const u32x4 w = *reinterpret_cast<const u32x4 *>(row + c);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      m = fmaxf(m, fmaxf(__builtin_fabsf(__uint_as_float(w[i] << 16)),
                         __builtin_fabsf(__uint_as_float(w[i] & 0xFFFF0000u))));
  }
  m = wave_max(m);
  if (wide) {   // every wave of the block is in this branch (wide is uniform)
    if (lane == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  }
  const int s = m > 0.0f ? exponent_of(m) - 15 : 0;
  for (int64_t c = t0 * 8; c < H; c += step) {
    const u32x4 w = *reinterpret_cast<const u32x4 *>(row + c);
    f16x8 h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[2 * i] = (_Float16)__builtin_ldexpf(__uint_as_float(w[i] << 16), -s);
      h[2 * i + 1] = (_Float16)__builtin_ldexpf(__uint_as_float(w[i] & 0xFFFF0000u), -s);
    }
    *reinterpret_cast<f16x8 *>(x16 + r * H + c) = h;
  }
  if (t0 == 0) xshift[r] = s;
}

// A dropped slot (id outside 0..E-1: its Y row was never written) is not
// added; a token without kept slots gets 0.
__global__ __launch_bounds__(256) void combine_kernel(const float *ypair, int64_t T, int64_t H,
                                                      int k, const int32_t *ids, int E, void *y,
                                                      OutType t) {
  const int64_t groups = T * (H / 4);
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < groups;
       g += (int64_t)gridDim.x * 256) {
    const int64_t tok = g / (H / 4), c = (g - tok * (H / 4)) * 4;
    f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
    bool any = false;
    for (int j = 0; j < k; ++j) {
      if ((unsigned)ids[tok * k + j] >= (unsigned)E) continue;
      const f32x4 v = *reinterpret_cast<const f32x4 *>(ypair + (tok * k + j) * H + c);
      s = any ? s + v : v;
      any = true;
    }
    if (t == OutType::F32) {
      *reinterpret_cast<f32x4 *>(static_cast<float *>(y) + tok * H + c) = s;
    } else {
      u32x2 w;
      w[0] = f32_to_bf16_bits(s[0]) | (f32_to_bf16_bits(s[1]) << 16);
      w[1] = f32_to_bf16_bits(s[2]) | (f32_to_bf16_bits(s[3]) << 16);
      *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(y) + tok * H + c) = w;
    }
  }
}

}  // namespace

int gemm_block_rows(int64_t rows_hint) {
  if (rows_hint <= 16) return 16;
  if (rows_hint <= 32) return 32;
  if (rows_hint <= 64) return 64;
  return 128;
}

hipError_t launch_gemm(Epi epi, const GemmArgs &a, int bm, hipStream_t s) {
  switch (bm) {
    case 16: return launch_cfg<1, 4, 1>(epi, a, s);
    case 32: return launch_cfg<1, 4, 2>(epi, a, s);
    case 64: return launch_cfg<2, 4, 4>(epi, a, s);
    default: return launch_cfg<4, 4, 8>(epi, a, s);
  }
}

hipError_t launch_moe_plan(const int32_t *offsets, int E, int bm, int4 *mblocks,
                           int32_t *n_mblocks, int bm2, int4 *mblocks2, int32_t *n_mblocks2,
                           uint32_t *zero, int zero_words, hipStream_t s) {
  launch_kernel(moe_plan_kernel, dim3(1), dim3(1024), 0, s, offsets, E, bm, mblocks,
                     n_mblocks, bm2, mblocks2, n_mblocks2, zero, zero_words);
  return hipGetLastError();
}

hipError_t launch_moe_prep(const uint16_t *x, int64_t T, int64_t H, _Float16 *x16,
                           int32_t *xshift, const int32_t *offsets, int E, int bm,
                           int4 *mblocks, int32_t *n_mblocks, int bm2, int4 *mblocks2,
                           int32_t *n_mblocks2, uint32_t *zero, int64_t zero_words,
                           hipStream_t s) {
  const int wide = T <= 1024;
  const int64_t blocks = (wide ? T : (T + 3) / 4) + 1;
  launch_kernel(moe_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, T, H, x16, xshift,
                offsets, E, bm, mblocks, n_mblocks, bm2, mblocks2, n_mblocks2, zero, zero_words,
                wide);
  return hipGetLastError();
}

hipError_t launch_combine(const float *ypair, int64_t T, int64_t H, int k, const int32_t *ids,
                          int E, void *y, OutType t, hipStream_t s) {
  int64_t blocks = (T * (H / 4) + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  launch_kernel(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, s, ypair, T, H, k, ids, E,
                y, t);
  return hipGetLastError();
}

}  // namespace nvfp4

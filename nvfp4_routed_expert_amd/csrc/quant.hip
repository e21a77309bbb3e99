// NVFP4 quantisation, debug dequantisation and activation preparation.
//
// Quantisation is an encoding: its fp32 steps are fixed (one tensor decode
// scale g = amax / 2688, per 16-block E4M3 scale amax_b / (6 g) rounded to
// nearest-even and saturated at 448, per element E2M1 of x * (1 / (s g))
// rounded to nearest-even and saturated at 6).  The pages name NVFP4 with
// 16-element blocks and E4M3 scales only by reference to the checkpoint
// formats (Qwen3.8-Flash-Next-NVFP4-SSD-Stream model card, "What this model
// is"); the rounding rules are this library's documented reading.
#include "common.h"
#include "kernels.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void load8(const void *base, InType t, int64_t idx, float (&v)[8]) {
  if (t == InType::BF16) {
    const u32x4 w = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(base) + idx);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float *p = static_cast<const float *>(base) + idx;
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
}

// Max over the workgroup (256 threads); every thread gets the result.
__device__ float block_max(float v, float *lds4) {
  v = wave_max(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds4[wave] = v;
  __syncthreads();
  float m = lds4[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) m = fmaxf(m, lds4[i]);
  __syncthreads();
  return m;
}

// g from the caller, or from the maximum of `n` stored maxima.
__device__ float resolve_global(const float *amax_src, int n, const float *g_given, float *lds4) {
  if (g_given) return *g_given;
  float m = 0.0f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) m = fmaxf(m, amax_src[i]);
  return global_from_amax(block_max(m, lds4));
}

// Groups of 8 elements, kAmaxBatch of them per thread and step with every
// load issued before the first is used.
constexpr int kAmaxBatch = 8;
__global__ __launch_bounds__(kThreads) void amax_partials_kernel(
    const void *x, InType t, int64_t rows, int64_t cols, int64_t ld, float *partials) {
  __shared__ float lds[4];
  const int64_t gpr = cols / 8, groups = rows * gpr;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  float m = 0.0f;
  for (int64_t g0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; g0 < groups;
       g0 += stride * kAmaxBatch) {
    float v[kAmaxBatch][8];
#pragma unroll
    for (int u = 0; u < kAmaxBatch; ++u) {
      const int64_t g = g0 + u * stride;
      const int64_t gg = g < groups ? g : g0;   // past the end: a valid group again
      const int64_t r = gg / gpr, c = (gg - r * gpr) * 8;
      load8(x, t, r * ld + c, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kAmaxBatch; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, __builtin_fabsf(v[u][i]));
  }
  m = block_max(m, lds);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

__global__ __launch_bounds__(kThreads) void quantize_kernel(
    const void *x, InType t, int64_t rows, int64_t cols, int64_t ld, uint8_t *codes,
    uint8_t *scales, const float *amax_src, int n_amax, const float *g_given, float *g_out) {
  __shared__ float lds[4];
  const float g = resolve_global(amax_src, n_amax, g_given, lds);
  const int64_t bpr = cols / 16, blocks = rows * bpr;
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < blocks;
       b += (int64_t)gridDim.x * kThreads) {
    const int64_t r = b / bpr, cb = b - r * bpr;
    float v[16];
    float (&v0)[8] = *reinterpret_cast<float (*)[8]>(&v[0]);
    float (&v1)[8] = *reinterpret_cast<float (*)[8]>(&v[8]);
    load8(x, t, r * ld + cb * 16, v0);
    load8(x, t, r * ld + cb * 16 + 8, v1);
    const Block16 q = quantize_block16(v, g);
    u32x2 w;
    w[0] = q.lo;
    w[1] = q.hi;
    *reinterpret_cast<u32x2 *>(codes + r * (cols / 2) + cb * 8) = w;
    scales[r * bpr + cb] = (uint8_t)q.scale;
  }
  if (g_out && blockIdx.x == 0 && threadIdx.x == 0) *g_out = g;
}

// out[r][c] (fp32) = e2m1 * e4m3 * g.  The product e2m1 * e4m3 is formed in
// fp16 by the same packed conversion the GEMMs use (exact), then one fp32
// multiply by g rounds it once.
__global__ __launch_bounds__(kThreads) void dequantize_kernel(
    const uint8_t *codes, const uint8_t *scales, const float *gp, int64_t rows,
    int64_t cols, float *out) {
  const float g = *gp;
  const int64_t gpr = cols / 8, groups = rows * gpr;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < groups;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t r = i / gpr, c8 = i - r * gpr;
    const uint32_t word = *reinterpret_cast<const uint32_t *>(codes + r * (cols / 2) + c8 * 4);
    const uint32_t sbyte = scales[r * (cols / 16) + c8 / 2];
    f16x2 s0, s1;
    e4m3x2_to_f16_pairs(sbyte, s0, s1);
    const f16x8 d = dequant8_f16(word, s0);
    f32x4 a, b;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a[j] = (float)d[j] * g;
      b[j] = (float)d[4 + j] * g;
    }
    float *o = out + r * cols + c8 * 8;
    *reinterpret_cast<f32x4 *>(o) = a;
    *reinterpret_cast<f32x4 *>(o + 4) = b;
  }
}

// SHIFT mode for few rows: one workgroup per row (the row maximum reduced
// over its four waves), so a long row is not one wavefront's serial loop.
__global__ __launch_bounds__(kThreads) void row_shift_wide_kernel(const uint16_t *x, int64_t cols,
                                                                 _Float16 *out, int32_t *shift) {
  __shared__ float wmax[kThreads / 64];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  const uint16_t *row = x + r * cols;
  float m = 0.0f;
  for (int64_t c = tid * 8; c < cols; c += kThreads * 8) {
    float v[8];
    load8(row, InType::BF16, c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, __builtin_fabsf(v[i]));
  }
  m = wave_max(m);
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const int s = m > 0.0f ? exponent_of(m) - 15 : 0;
  for (int64_t c = tid * 8; c < cols; c += kThreads * 8) {
    float v[8];
    load8(row, InType::BF16, c, v);
    f16x8 h;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (_Float16)__builtin_ldexpf(v[i], -s);
    *reinterpret_cast<f16x8 *>(out + r * cols + c) = h;
  }
  if (tid == 0) shift[r] = s;
}

// One wavefront per row.
__global__ __launch_bounds__(kThreads) void row_prep_kernel(
    const uint16_t *x, int64_t rows, int64_t cols, PrepMode mode, _Float16 *out,
    int32_t *shift, const float *amax_src, int n_amax, const float *g_given,
    float *g_out, float *g_out2) {
  __shared__ float lds[4];
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (mode == PrepMode::SHIFT) {
    if (r >= rows) return;
    const uint16_t *row = x + r * cols;
    float m = 0.0f;
    for (int64_t c = lane * 8; c < cols; c += 512) {
      float v[8];
      load8(row, InType::BF16, c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, __builtin_fabsf(v[i]));
    }
    m = wave_max(m);
    // bf16 values scaled so the row maximum has exponent 15 stay <= 65280
    // and are exact in fp16 down to 2^-32 of the row maximum.
    const int s = m > 0.0f ? exponent_of(m) - 15 : 0;
    for (int64_t c = lane * 8; c < cols; c += 512) {
      float v[8];
      load8(row, InType::BF16, c, v);
      f16x8 h;
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = (_Float16)__builtin_ldexpf(v[i], -s);
      *reinterpret_cast<f16x8 *>(out + r * cols + c) = h;
    }
    if (lane == 0) shift[r] = s;
    return;
  }
  // QUANT: every wave needs g before its row (all threads take part).
  const float g = resolve_global(amax_src, n_amax, g_given, lds);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (g_out) *g_out = g;
    if (g_out2) *g_out2 = g;
  }
  if (r >= rows) return;
  const uint16_t *row = x + r * cols;
  // up to kPrepSteps blocks of 16 per lane: all loads first, then the blocks
  constexpr int kPrepSteps = 4;
  for (int64_t c0 = lane * 16; c0 < cols; c0 += 1024 * kPrepSteps) {
    u32x4 raw[kPrepSteps][2];
#pragma unroll
    for (int st = 0; st < kPrepSteps; ++st) {
      const int64_t c = c0 + st * 1024;
      if (c < cols) {
        raw[st][0] = *reinterpret_cast<const u32x4 *>(row + c);
        raw[st][1] = *reinterpret_cast<const u32x4 *>(row + c + 8);
      }
    }
#pragma unroll
    for (int st = 0; st < kPrepSteps; ++st) {
      const int64_t c = c0 + st * 1024;
      if (c >= cols) break;
      float v[16];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[8 * h + 2 * i] = __uint_as_float(raw[st][h][i] << 16);
          v[8 * h + 2 * i + 1] = __uint_as_float(raw[st][h][i] & 0xFFFF0000u);
        }
      const Block16 q = quantize_block16(v, g);
      // the exact fp16 products e2m1 * e4m3, as the GEMM operands expect
      f16x2 s0, s1;
      e4m3x2_to_f16_pairs(q.scale, s0, s1);
      const f16x8 h0 = dequant8_f16(q.lo, s0);
      const f16x8 h1 = dequant8_f16(q.hi, s0);
      *reinterpret_cast<f16x8 *>(out + r * cols + c) = h0;
      *reinterpret_cast<f16x8 *>(out + r * cols + c + 8) = h1;
    }
  }
}

int grid_for(int64_t work_items, int per_block) {
  int64_t g = (work_items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > 4096) g = 4096;
  return (int)g;
}

}  // namespace

int amax_partials_grid(int64_t rows, int64_t cols) {
  int64_t g = (rows * (cols / 8) + kThreads * 8 - 1) / (kThreads * 8);
  if (g < 1) g = 1;
  if (g > kMaxPartials) g = kMaxPartials;
  return (int)g;
}

hipError_t launch_amax_partials(const void *x, InType t, int64_t rows, int64_t cols,
                                int64_t ld, float *partials, int n_partials,
                                hipStream_t s) {
  launch_kernel(amax_partials_kernel, dim3(n_partials), dim3(kThreads), 0, s, x, t,
                     rows, cols, ld, partials);
  return hipGetLastError();
}

hipError_t launch_quantize(const void *x, InType t, int64_t rows, int64_t cols,
                           int64_t ld, uint8_t *codes, uint8_t *scales,
                           const float *amax_src, int n_amax, const float *g_given,
                           float *g_out, hipStream_t s) {
  launch_kernel(quantize_kernel, dim3(grid_for(rows * (cols / 16), kThreads)),
                     dim3(kThreads), 0, s, x, t, rows, cols, ld, codes, scales, amax_src,
                     n_amax, g_given, g_out);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t *codes, const uint8_t *scales, const float *g,
                             int64_t rows, int64_t cols, float *out, hipStream_t s) {
  launch_kernel(dequantize_kernel, dim3(grid_for(rows * (cols / 8), kThreads)),
                     dim3(kThreads), 0, s, codes, scales, g, rows, cols, out);
  return hipGetLastError();
}

hipError_t launch_row_prep(const uint16_t *x, int64_t rows, int64_t cols, PrepMode mode,
                           _Float16 *out, int32_t *shift, const float *amax_src,
                           int n_amax, const float *g_given, float *g_out,
                           float *g_out2, hipStream_t s) {
  static_assert(kThreads == 256, "row_shift_wide_kernel reduces four waves");
  if (mode == PrepMode::SHIFT && rows <= 1024) {   // few rows: a workgroup each
    launch_kernel(row_shift_wide_kernel, dim3((unsigned)rows), dim3(kThreads), 0, s, x, cols, out,
                  shift);
    return hipGetLastError();
  }
  const int64_t blocks = (rows + 3) / 4;
  launch_kernel(row_prep_kernel, dim3((unsigned)(blocks < 1 ? 1 : blocks)),
                     dim3(kThreads), 0, s, x, rows, cols, mode, out, shift, amax_src,
                     n_amax, g_given, g_out, g_out2);
  return hipGetLastError();
}

}  // namespace nvfp4

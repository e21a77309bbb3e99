// The BF16 shared expert beside the routed NVFP4 experts (Qwen3.8-Flash-Next-
// NVFP4-SSD-Stream model card, "What this model is": shared experts stay
// BF16; DwarfStar page: shared experts are replicated on every device):
//   h = bf16( silu(x Wg^T) * (x Wu^T) ),   y (+)= h Wd^T
// The three products run as bf16 MFMA partial sums (router.hip); these two
// streaming kernels add the parts in part order and apply the SiLU * up
// epilogue (the same fp32 steps as the routed FFN's) and the final sum.
#include "common.h"
#include "kernels.h"

namespace nvfp4 {
namespace {

typedef __attribute__((ext_vector_type(4))) float f4;

constexpr int kSharedThreads = 256;

// Thread: 8 consecutive i of token t.  I % 8 == 0.
__global__ __launch_bounds__(kSharedThreads) void shared_h_kernel(const float *gp, int parts,
                                                                   int64_t T, int64_t I,
                                                                   int64_t part_stride,
                                                                   uint16_t *h) {
  const int64_t idx = (int64_t)blockIdx.x * kSharedThreads + threadIdx.x;
  const int64_t n8 = T * I / 8;
  if (idx >= n8) return;
  const int64_t t = idx / (I / 8), i0 = (idx % (I / 8)) * 8;
  const float *g = gp + t * 2 * I + i0;
  const float *u = g + I;
  f4 G[2], U[2];
  G[0] = *reinterpret_cast<const f4 *>(g);
  G[1] = *reinterpret_cast<const f4 *>(g + 4);
  U[0] = *reinterpret_cast<const f4 *>(u);
  U[1] = *reinterpret_cast<const f4 *>(u + 4);
  for (int s = 1; s < parts; ++s) {
    const int64_t o = s * part_stride;
    G[0] += *reinterpret_cast<const f4 *>(g + o);
    G[1] += *reinterpret_cast<const f4 *>(g + o + 4);
    U[0] += *reinterpret_cast<const f4 *>(u + o);
    U[1] += *reinterpret_cast<const f4 *>(u + o + 4);
  }
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t b[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = 2 * j + q;
      const float gv = G[e >> 2][e & 3], uv = U[e >> 2][e & 3];
      b[q] = f32_to_bf16_bits(gv / (1.0f + expf(-gv)) * uv);
    }
    w[j] = b[0] | (b[1] << 16);
  }
  typedef __attribute__((ext_vector_type(4))) uint32_t u4;
  *reinterpret_cast<u4 *>(h + t * I + i0) = u4{w[0], w[1], w[2], w[3]};
}

// Thread: 4 consecutive outputs.  (T * H) % 4 == 0.
__global__ __launch_bounds__(kSharedThreads) void shared_out_kernel(const float *yp, int parts,
                                                                     int64_t n, int accumulate,
                                                                     void *y, OutType ot) {
  const int64_t idx = (int64_t)blockIdx.x * kSharedThreads + threadIdx.x;
  if (idx * 4 >= n) return;
  const int64_t o = idx * 4;
  f4 v = *reinterpret_cast<const f4 *>(yp + o);
  for (int s = 1; s < parts; ++s) v += *reinterpret_cast<const f4 *>(yp + s * n + o);
  if (ot == OutType::F32) {
    f4 *p = reinterpret_cast<f4 *>(static_cast<float *>(y) + o);
    if (accumulate) v = *p + v;
    *p = v;
  } else {
    uint2 *p = reinterpret_cast<uint2 *>(static_cast<uint16_t *>(y) + o);
    if (accumulate) {
      const uint2 old = *p;
      v[0] = bf16_bits_to_f32(old.x & 0xFFFFu) + v[0];
      v[1] = bf16_bits_to_f32(old.x >> 16) + v[1];
      v[2] = bf16_bits_to_f32(old.y & 0xFFFFu) + v[2];
      v[3] = bf16_bits_to_f32(old.y >> 16) + v[3];
    }
    *p = make_uint2(f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16),
                    f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16));
  }
}

}  // namespace

hipError_t launch_shared_h(const float *gp, int parts, int64_t T, int64_t I, uint16_t *h,
                           hipStream_t s) {
  if (I % 8 != 0) return hipErrorInvalidValue;
  const int64_t n8 = T * I / 8;
  launch_kernel(shared_h_kernel, dim3((unsigned)((n8 + kSharedThreads - 1) / kSharedThreads)),
                dim3(kSharedThreads), 0, s, gp, parts, T, I, T * 2 * I, h);
  return hipGetLastError();
}

hipError_t launch_shared_out(const float *yp, int parts, int64_t T, int64_t H, bool accumulate,
                             void *y, OutType t, hipStream_t s) {
  const int64_t n = T * H;
  if (n % 4 != 0) return hipErrorInvalidValue;
  launch_kernel(shared_out_kernel,
                dim3((unsigned)((n / 4 + kSharedThreads - 1) / kSharedThreads)),
                dim3(kSharedThreads), 0, s, yp, parts, n, accumulate ? 1 : 0, y, t);
  return hipGetLastError();
}

}  // namespace nvfp4

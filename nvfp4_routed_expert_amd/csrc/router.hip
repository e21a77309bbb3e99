// BF16 products x . W^T as K-split fp32 partial sums, for the parts of the
// model that stay BF16 beside the NVFP4 routed experts (Qwen3.8-Flash-Next-
// NVFP4-SSD-Stream model card, "What this model is"): the router (logits
// l[t][e] = x_t . R_e, R [E, H]; the top-k kernels add the parts in part
// order while they load the logits, route.hip LogitSrc) and the shared
// expert (shared.hip).  W is one row-major [N, K] matrix, or two stacked
// ones (rows n < N0 from the first, the rest from the second: gate over up).
//
// A wavefront computes a tile of 16 MS tokens x 16 NB experts over one K
// part with v_mfma_f32_16x16x32_bf16 (MS = NB = 1 below 64 tokens, else 2),
// one wavefront per workgroup so the tiles spread over every CU.  Both
// operands come straight from global memory into the MFMA fragments (no
// LDS), several K steps' loads at a time: lane l reads 16 bytes (8 bf16
// along K) of row l % 16 at K offset 8 (l / 16) for each 16-row subtile, so
// the four lanes of a row cover 64 contiguous bytes and two K steps a full
// 128-byte line.  Products of two bf16 values are exact in fp32; the sums are
// fp32.  K is cut into up to four parts when the tiles alone leave CUs idle,
// so that enough wavefronts stream R at once.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace nvfp4 {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kRouterWaves = 1;       // one tile per workgroup: the tiles spread over every CU
constexpr int kRouterTargetWaves = 1024;

// 16 bytes at p (always a valid address: rows past the end read row 0),
// zero where !ok
__device__ __forceinline__ bf16x8 load8(const uint16_t *p, bool ok) {
  u32x4 v = *reinterpret_cast<const u32x4 *>(p);
  const u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, ok ? v : z);
}

template <int MS, int NB>
__global__ __launch_bounds__(64 * kRouterWaves) void bf16_partials_kernel(
    const uint16_t *x, const uint16_t *W0, const uint16_t *W1, int N0, int T, int H, int E,
    int kpart, int n_tb, int n_eb, int n_items, float *partial) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * kRouterWaves + (threadIdx.x >> 6);
  if (item >= n_items) return;
  // item = (kz * n_tb + tb) * n_eb + eb: the waves of a workgroup share x rows
  const int eb = item % n_eb;
  const int rest = item / n_eb;
  const int tb = rest % n_tb;
  const int kz = rest / n_tb;
  const int lr = lane & 15, lg = lane >> 4;
  const int k0 = kz * kpart;
  const int k1 = min(H, k0 + kpart);
  const uint16_t *xa[MS];
  const uint16_t *rb[NB];
  bool xok[MS], rok[NB];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    const int t = tb * 16 * MS + ms * 16 + lr;
    xok[ms] = t < T;
    xa[ms] = x + (int64_t)(xok[ms] ? t : 0) * H + 8 * lg;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int e = eb * 16 * NB + nb * 16 + lr;
    rok[nb] = e < E;
    const int ec = rok[nb] ? e : 0;
    rb[nb] = ec < N0 ? W0 + (int64_t)ec * H + 8 * lg : W1 + (int64_t)(ec - N0) * H + 8 * lg;
  }
  f32x4 acc[MS][NB];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[ms][nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // 64-wide steps (two MFMAs each, so every row's loads cover whole lines),
  // in rounds of up to 8 / MS steps whose loads are all issued first
  constexpr int U = 8 / MS;
  const int n64 = (k1 - k0) / 64;
  int k = k0;
  auto steps = [&](auto n_const) {
    constexpr int NS = decltype(n_const)::value;
    bf16x8 a[NS][2][MS], b[NS][2][NB];
#pragma unroll
    for (int u = 0; u < NS; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) a[u][h][ms] = load8(xa[ms] + k + 64 * u + 32 * h, xok[ms]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) b[u][h][nb] = load8(rb[nb] + k + 64 * u + 32 * h, rok[nb]);
      }
#pragma unroll
    for (int u = 0; u < NS; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            acc[ms][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][h][ms], b[u][h][nb],
                                                                  acc[ms][nb], 0, 0, 0);
    k += 64 * NS;
  };
  int i = 0;
  for (; i + U <= n64; i += U) steps(std::integral_constant<int, U>{});
  if constexpr (U > 2)
    for (; i + 2 <= n64; i += 2) steps(std::integral_constant<int, 2>{});
  for (; i < n64; ++i) steps(std::integral_constant<int, 1>{});
  if (k < k1) {   // a last 32-wide step (H % 64 == 32)
    bf16x8 a0[MS], b0[NB];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) a0[ms] = load8(xa[ms] + k, xok[ms]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) b0[nb] = load8(rb[nb] + k, rok[nb]);
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[ms][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[ms], b0[nb], acc[ms][nb], 0, 0, 0);
  }
  // lane holds tokens 4 lg + j of each subtile, expert lr of each block
  float *out = partial + (int64_t)kz * T * E;
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = tb * 16 * MS + ms * 16 + 4 * lg + j;
      if (t >= T) continue;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int e = eb * 16 * NB + nb * 16 + lr;
        if (e < E) out[(int64_t)t * E + e] = acc[ms][nb][j];
      }
    }
}

}  // namespace

Bf16Plan bf16_plan(int64_t T, int64_t H, int64_t E) {
  Bf16Plan p;
  p.ms = T >= 64 ? 2 : 1;
  p.nb = p.ms;
  const int64_t n_tb = (T + 16 * p.ms - 1) / (16 * p.ms);
  const int64_t n_eb = (E + 16 * p.nb - 1) / (16 * p.nb);
  const int64_t items = n_tb * n_eb;
  int64_t parts = (kRouterTargetWaves + items - 1) / items;
  if (parts > kMaxLogitParts) parts = kMaxLogitParts;   // the top-k adds them while loading
  if (parts > H / 64) parts = H / 64;
  if (parts < 1) parts = 1;
  // a part is a whole number of 64-wide steps (the last one may be shorter)
  p.kpart = (int)(((H + parts - 1) / parts + 63) / 64 * 64);
  p.parts = (int)((H + p.kpart - 1) / p.kpart);
  p.partial_floats = (size_t)p.parts * T * E;
  return p;
}

hipError_t launch_bf16_partials(const uint16_t *x, const uint16_t *W0, const uint16_t *W1,
                                int64_t N0, int64_t T, int64_t H, int64_t E, const Bf16Plan &p,
                                float *partial, hipStream_t s) {
  if (!W1) N0 = E;
  if (H % 32 != 0 || p.kpart % 64 != 0) return hipErrorInvalidValue;
  const int n_tb = (int)((T + 16 * p.ms - 1) / (16 * p.ms));
  const int n_eb = (int)((E + 16 * p.nb - 1) / (16 * p.nb));
  const int64_t n_items = (int64_t)n_tb * n_eb * p.parts;
  if (n_items > INT32_MAX - kRouterWaves) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((n_items + kRouterWaves - 1) / kRouterWaves)), block(64 * kRouterWaves);
  const int a[] = {(int)T, (int)H, (int)E, p.kpart, n_tb, n_eb, (int)n_items};
  switch (p.ms) {
    case 1:
      launch_kernel(bf16_partials_kernel<1, 1>, grid, block, 0, s, x, W0, W1, (int)N0, a[0], a[1],
                    a[2], a[3], a[4], a[5], a[6], partial);
      break;
    default:
      launch_kernel(bf16_partials_kernel<2, 2>, grid, block, 0, s, x, W0, W1, (int)N0, a[0], a[1],
                    a[2], a[3], a[4], a[5], a[6], partial);
      break;
  }
  return hipGetLastError();
}

}  // namespace nvfp4

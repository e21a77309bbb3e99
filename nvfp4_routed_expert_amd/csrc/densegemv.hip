// Dense NVFP4 GEMV for a few rows (M <= 32): the decode form of a dense
// NVFP4 MLP or linear (Eider page, "Qwen3.8 27B": NVFP4 for most MLP
// weights), where the weight stream is the whole cost and every row of the
// batch must share it.
//
// Weights leave HBM as whole 128-byte lines: a K chunk is 256 elements, so
// each weight row's chunk is one line of codes plus 16 scale bytes, and a
// direct global-to-LDS load of 1 KB covers eight rows' lines.  (Loading
// weights straight into MFMA fragments gives each row only 32-64 bytes per
// instruction, which streams far below the HBM rate.)  A wave reads its
// fragments back from LDS, dequantises them in registers (E2M1 -> fp16 by
// the packed converter, times the E4M3 block scale in packed fp16: exact)
// and multiplies them with v_mfma_f32_16x16x32_f16 against the fp16
// activation rows, which are staged in the same ring.  One weight stream
// serves all M rows (one or two 16-row subtiles).
//
// A tile is 128 weight rows: for the gate/up pair each of the four waves
// owns 16 gate rows and the 16 up rows of the same h columns (64 h columns
// per tile), otherwise 32 output columns.  The work is the sequence of
// (tile, chunk) units, tile-major; a persistent grid of G workgroups (two
// per CU, or one with two 16-row subtiles) gives workgroup g the contiguous
// units [g U / G, (g + 1) U / G), so every SIMD streams the same amount
// however few the tiles are, and the LDS ring stays full across tile
// boundaries (a workgroup pays the HBM latency once).  At the end of each
// tile, or of its range, a workgroup writes its raw sums for that tile as a
// partial; the reduce kernel adds the partials of each tile in workgroup
// order (deterministic) and applies the epilogue.
//
// K permutation: in a chunk, lane group g = lane / 16 supplies the 64
// elements 64 g .. 64 g + 63 over the eight 32-wide MFMA steps (8 per step),
// for both operands; a lane then needs 32 code bytes and 4 scale bytes of
// its weight row per chunk.  LDS pieces of 16 bytes are XOR-swizzled by the
// row so that the 16 rows of a fragment spread over the banks.
#include <type_traits>

#include "common.h"
#include "kernels.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

namespace nvfp4 {
namespace {

constexpr int kDC = 256;                      // K per chunk
constexpr int kDWaves = 4;
constexpr int kDRows = 32 * kDWaves;          // weight rows per tile
constexpr int kDCodeRow = kDC / 2;            // code bytes per row and chunk (one line)
constexpr int kDScaleRow = kDC / 16;          // scale bytes per row and chunk
constexpr int kDCUs = 256;

template <int MS>
struct DenseCfg {
  // two-stage rings: three workgroups with one 16-row subtile (26 KB
  // stages) or two with two (34 KB stages) share a CU
  static constexpr int STAGES = 2;
  static constexpr int PER_CU = MS == 1 ? 3 : 2;
  static constexpr int MP = 16 * MS;                        // activation rows staged
  static constexpr int B_BYTES = kDRows * kDCodeRow;        // 16 KB
  static constexpr int S_BYTES = kDRows * kDScaleRow;       // 2 KB
  static constexpr int A_BYTES = MP * kDC * 2;              // 8 or 16 KB
  static constexpr int STAGE = B_BYTES + S_BYTES + A_BYTES;
  static constexpr int B_LOADS = B_BYTES / 1024 / kDWaves;  // 16-byte lanes, 1 KB each
  static constexpr int S_LOADS = S_BYTES / 256 / kDWaves;   // 4-byte lanes, 256 B each
  static constexpr int A_LOADS = A_BYTES / 1024 / kDWaves;
  static constexpr int LOADS = B_LOADS + S_LOADS + A_LOADS; // per wave and chunk
  static_assert(B_BYTES % (1024 * kDWaves) == 0 && S_BYTES % (256 * kDWaves) == 0 &&
                    A_BYTES % (1024 * kDWaves) == 0,
                "stages split evenly over the waves");
};

typedef __attribute__((address_space(3))) void *lds_ptr_t;

template <Epi EPI>
constexpr int dense_cols() { return EPI == Epi::SWIGLU ? 16 * kDWaves : 32 * kDWaves; }
// raw-sum columns of a tile in a partial (gate/up: the gate then the up sums)
constexpr int kDPartCols = 2 * 16 * kDWaves;

// Unit split: workgroup g owns units [first(g), first(g + 1)).
struct StreamSplit {
  int64_t units;   // tiles * chunks per tile
  int grid;        // G
  int nch;         // chunks per tile (K / 256)
  int slots;       // most tiles a workgroup touches
};
__host__ __device__ inline int64_t unit_first(const StreamSplit &s, int64_t g) {
  return g * s.units / s.grid;
}
// the workgroup whose range holds unit u: the largest g with first(g) <= u
__host__ __device__ inline int64_t unit_owner(const StreamSplit &s, int64_t u) {
  return ((u + 1) * s.grid + s.units - 1) / s.units - 1;
}

// E2M1 codes of one word -> eight exact bf16 products with the block scale
// (through fp32: gfx950 has no packed bf16 multiply; e2m1 * e4m3 has at most
// six significant bits, so every step is exact)
__device__ __forceinline__ bf16x8 dequant8_bf16(uint32_t word, float s) {
  const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0);
  const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1);
  const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2);
  const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3);
  bf16x8 r;
  r[0] = (__bf16)(v0[0] * s); r[1] = (__bf16)(v0[1] * s);
  r[2] = (__bf16)(v1[0] * s); r[3] = (__bf16)(v1[1] * s);
  r[4] = (__bf16)(v2[0] * s); r[5] = (__bf16)(v2[1] * s);
  r[6] = (__bf16)(v3[0] * s); r[7] = (__bf16)(v3[1] * s);
  return r;
}

// BF: the activation rows are bf16 as given (a dense MLP's x and h), the
// weights are dequantised to bf16 and multiplied by v_mfma_f32_16x16x32_bf16;
// the products are the same exact values as in the fp16 form, which needs
// its operand rows converted to fp16 with a power-of-two row shift by
// passes of their own.
template <int MS, Epi EPI, bool BF>
__global__ __launch_bounds__(64 * kDWaves, MS == 1 ? 3 : 2) void dense_gemv_kernel(
    const GemmArgs p, int M, const StreamSplit sk, float *partial) {
  using C = DenseCfg<MS>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::STAGES * C::STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int K = p.K, N = p.N;
  constexpr int kCols = dense_cols<EPI>();
  const int64_t u0 = unit_first(sk, blockIdx.x), u1 = unit_first(sk, blockIdx.x + 1);
  if (u0 >= u1) return;   // (more workgroups than units: whole workgroup, uniform)
  const int t0 = (int)(u0 / sk.nch);

  // ---- loader state -----------------------------------------------------------
  // Tile-local weight row r: wave r / 32, fragment (r / 16) & 1, row r % 16.
  // SWIGLU: fragment 0 is the gate row and fragment 1 the up row of h column
  // t * 64 + 16 wave + r % 16; otherwise output row t * 128 + r.  Rows past N
  // reread row N - 1.
  const int64_t code_row = K / 2, scale_row = K / 16;
  auto row_of = [&](int t, int r, int &mat) {
    int row;
    if constexpr (EPI == Epi::SWIGLU) {
      mat = (r >> 4) & 1;
      row = t * kCols + 16 * (r >> 5) + (r & 15);
    } else {
      mat = 0;
      row = t * kCols + r;
    }
    return row < N ? row : N - 1;
  };
  // codes: instruction q of wave w (q = B_LOADS w + j) fills LDS rows
  // 8 q .. 8 q + 7; lane l writes piece l % 8 of row 8 q + l / 8 and fetches
  // piece (l % 8) ^ (row % 8) of that row's line.  scales: instruction q
  // fills 256 bytes = rows 16 q .. 16 q + 15; lane l writes bytes 4 (l % 4)
  // .. of row 16 q + l / 4.  activations: instruction q fills rows 2 q,
  // 2 q + 1 (512 bytes each); lane l writes piece l % 32 of row 2 q + l / 32
  // and fetches piece (l % 32) ^ (row % 8); rows past M reread row M - 1
  // (results discarded).  (Fixed-size arrays: with sizes that depend on the
  // template arguments the host pass of this compiler drops the kernel's
  // launch stub.)
  static_assert(C::B_LOADS <= 4 && C::S_LOADS <= 2 && C::A_LOADS <= 4, "loader arrays");
  int crow[4], spiece[4];
#pragma unroll
  for (int j = 0; j < C::B_LOADS; ++j) {
    crow[j] = 8 * (C::B_LOADS * wave + j) + (lane >> 3);
    spiece[j] = 16 * ((lane & 7) ^ (crow[j] & 7));
  }
  int srow[2];
#pragma unroll
  for (int j = 0; j < C::S_LOADS; ++j) srow[j] = 16 * (C::S_LOADS * wave + j) + (lane >> 2);
  const _Float16 *asrc[4];
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j) {
    const int m = 2 * (C::A_LOADS * wave + j) + (lane >> 5);
    const int mm = m < M ? m : M - 1;
    int arow = p.a_rowmap ? p.a_rowmap[mm] : mm;
    arow = arow < 0 ? 0 : arow / (p.a_rowmap ? p.a_rowdiv : 1);   // (a dropped pair: row 0)
    asrc[j] = p.A + (int64_t)arow * p.lda + 8 * ((lane & 31) ^ (m & 7));
  }

  // Issue the loads of unit u (tile u / nch, chunk u % nch) into ring slot
  // (u - u0) % STAGES.
  auto load_unit = [&](int64_t u) {
    const int t = (int)(u / sk.nch), c = (int)(u - (int64_t)t * sk.nch);
    uint8_t *st = lds + (int)((u - u0) % C::STAGES) * C::STAGE;
#pragma unroll
    for (int j = 0; j < C::B_LOADS; ++j) {
      int mat;
      const int row = row_of(t, crow[j], mat);
      __builtin_amdgcn_global_load_lds(p.b_codes[mat] + row * code_row + (int64_t)c * kDCodeRow +
                                           spiece[j],
                                       (lds_ptr_t)(st + (C::B_LOADS * wave + j) * 1024), 16, 0,
                                       0);
    }
#pragma unroll
    for (int j = 0; j < C::S_LOADS; ++j) {
      int mat;
      const int row = row_of(t, srow[j], mat);
      __builtin_amdgcn_global_load_lds(p.b_scales[mat] + row * scale_row +
                                           (int64_t)c * kDScaleRow + 4 * (lane & 3),
                                       (lds_ptr_t)(st + C::B_BYTES +
                                                   (C::S_LOADS * wave + j) * 256),
                                       4, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < C::A_LOADS; ++j)
      __builtin_amdgcn_global_load_lds(asrc[j] + (int64_t)c * kDC,
                                       (lds_ptr_t)(st + C::B_BYTES + C::S_BYTES +
                                                   (C::A_LOADS * wave + j) * 1024),
                                       16, 0, 0);
  };

  f32x4 acc[MS][2];
  auto zero_acc = [&]() {
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
      for (int f = 0; f < 2; ++f) acc[ms][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  zero_acc();

  auto compute = [&](int64_t u) {
    const uint8_t *st = lds + (int)((u - u0) % C::STAGES) * C::STAGE;
    // this lane's 32 code bytes and 4 scale bytes of each fragment's row
    u32x4 cw[2][2];
    uint32_t sw[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int R = 32 * wave + 16 * f + lr;
      const uint8_t *row = st + R * kDCodeRow;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        cw[f][h] = *reinterpret_cast<const u32x4 *>(row + 16 * ((2 * lg + h) ^ (R & 7)));
      sw[f] = *reinterpret_cast<const uint32_t *>(st + C::B_BYTES + R * kDScaleRow + 4 * lg);
    }
    const uint8_t *abase = st + C::B_BYTES + C::S_BYTES;
    if constexpr (BF) {
      f32x2 sf[2][2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        sf[f][0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw[f], 1.0f, false);
        sf[f][1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw[f], 1.0f, true);
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        bf16x8 b[2];
#pragma unroll
        for (int f = 0; f < 2; ++f)
          b[f] = dequant8_bf16(cw[f][s >> 2][s & 3], sf[f][s >> 2][(s >> 1) & 1]);
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
          const int m = 16 * ms + lr;
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(abase + m * (kDC * 2) +
                                                             16 * ((8 * lg + s) ^ (m & 7)));
#pragma unroll
          for (int f = 0; f < 2; ++f)
            acc[ms][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[f], acc[ms][f], 0, 0, 0);
        }
      }
    } else {
      f16x2 sp[2][4];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        e4m3x2_to_f16_pairs(sw[f], sp[f][0], sp[f][1]);
        e4m3x2_to_f16_pairs(sw[f] >> 16, sp[f][2], sp[f][3]);
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        f16x8 b[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) b[f] = dequant8_f16(cw[f][s >> 2][s & 3], sp[f][s >> 1]);
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
          const int m = 16 * ms + lr;
          const f16x8 a = *reinterpret_cast<const f16x8 *>(abase + m * (kDC * 2) +
                                                           16 * ((8 * lg + s) ^ (m & 7)));
#pragma unroll
          for (int f = 0; f < 2; ++f)
            acc[ms][f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[f], acc[ms][f], 0, 0, 0);
        }
      }
    }
  };

  // raw sums of tile t into this workgroup's partial slot t - t0:
  // partial[g][slot][m][col], col = 0 .. 127 (gate/up: gate 0..63, up 64..127)
  auto store_partial = [&](int t) {
    float *part = partial + ((int64_t)blockIdx.x * sk.slots + (t - t0)) * 32 * kDPartCols;
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = 16 * ms + 4 * lg + j;
        if (m >= M) continue;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int col = EPI == Epi::SWIGLU ? 64 * f + 16 * wave + lr : 32 * wave + 16 * f + lr;
          part[m * kDPartCols + col] = acc[ms][f][j];
        }
      }
    }
  };

  // Ring of STAGES slots: units u + 1 .. u + STAGES - 1 in flight while unit
  // u is multiplied.  The wait before each barrier leaves only the newer
  // units' loads outstanding (STAGES - 2 units); the barrier then also
  // guarantees every wave is done with unit u - 1, whose slot the next loads
  // overwrite.  Past the range the last unit is requested again (a cache hit
  // into a slot nobody reads), so every wave always has the same number of
  // loads outstanding.
  const int64_t last = u1 - 1;
#pragma unroll
  for (int i = 0; i < C::STAGES - 1; ++i) load_unit(u0 + i <= last ? u0 + i : last);
  for (int64_t u = u0; u <= last; ++u) {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((C::STAGES - 2) * C::LOADS)
                 : "memory");
    load_unit(u + C::STAGES - 1 <= last ? u + C::STAGES - 1 : last);
    compute(u);
    const int t = (int)(u / sk.nch);
    if (u == last || (u + 1) % sk.nch == 0) {   // uniform: the tile ends here for this workgroup
      store_partial(t);
      zero_acc();
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Output element (m, n): the partials of tile t = n / kCols from the
// workgroups that own its units, added in workgroup order, then the epilogue
// (as the tile GEMM's).  Rows m are the dense rows (positions) 0..M-1.  The
// owners' partials are loaded kReduceBatch at a time before they are added
// (the same order), and the unit arithmetic runs in 32 bits when U32 (the
// host checks that units * grid fits): 64-bit divisions before every load
// serialised a tile's dozen round trips.
constexpr int kReduceBatch = 16;
// Lanes per output element: the gate/up tiles have two or three owners, the
// down and linear tiles a dozen or more (K is long), whose loads four lanes
// of a quad share (owners q, q + 4, ... in order per lane, then the quad's
// four sums added by two DPP exchanges: a fixed order, the same in each lane).
template <Epi EPI>
constexpr int reduce_lanes() { return EPI == Epi::SWIGLU ? 1 : 4; }
template <Epi EPI, bool U32>
__global__ __launch_bounds__(256) void dense_reduce_kernel(const GemmArgs p, int M,
                                                           const StreamSplit sk,
                                                           const float *partial) {
  constexpr int kCols = dense_cols<EPI>();
  constexpr int Q = reduce_lanes<EPI>();
  const int N = p.N;
  const int64_t tidx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t idx = tidx / Q;
  const int q = (int)(tidx - idx * Q);
  const bool in = idx < (int64_t)M * N;
  float amax = 0.0f;
  const int m = in ? (int)(idx / N) : 0, n = in ? (int)(idx - (int64_t)m * N) : 0;
  if constexpr (EPI == Epi::DOWN) {
    // row m of out as a token's row: zeros for a dropped token (no kept
    // position writes that row)
    if (in && q == 0 && p.drop_ids && (unsigned)p.drop_ids[m] >= (unsigned)p.n_experts) {
      if (p.out_type == OutType::F32)
        static_cast<float *>(p.out)[(int64_t)m * p.ldo + n] = 0.0f;
      else
        static_cast<uint16_t *>(p.out)[(int64_t)m * p.ldo + n] = 0;
    }
  }
  const int t = n / kCols, cl = n - t * kCols;
  const int pr = p.a_rowmap ? p.a_rowmap[m] : m;
  const bool valid = in && pr >= 0;   // (a dropped pair: no h row, no output)
  float s0 = 0.0f, s1 = 0.0f;
  if (valid) {
    const uint32_t units32 = (uint32_t)sk.units, grid32 = (uint32_t)sk.grid;
    const uint32_t nch32 = (uint32_t)sk.nch;
    auto owner = [&](int64_t u) -> int64_t {
      if constexpr (U32)
        return (int64_t)(((uint32_t)u + 1u) * grid32 + units32 - 1u) / units32 - 1;
      else
        return unit_owner(sk, u);
    };
    auto first_tile = [&](int64_t g) -> int {   // tile of workgroup g's first unit
      if constexpr (U32)
        return (int)((uint32_t)g * units32 / grid32 / nch32);
      else
        return (int)(unit_first(sk, g) / sk.nch);
    };
    const int64_t g_lo = owner((int64_t)t * sk.nch) + q;   // this lane's first owner
    const int64_t g_hi = owner((int64_t)t * sk.nch + sk.nch - 1);
    for (int64_t g0 = g_lo; g0 <= g_hi; g0 += (int64_t)kReduceBatch * Q) {
      float v0[kReduceBatch], v1[kReduceBatch];
#pragma unroll
      for (int u = 0; u < kReduceBatch; ++u) {
        const int64_t gu = g0 + (int64_t)u * Q;
        const int64_t g = gu <= g_hi ? gu : g0;   // (past the end: reread, unused)
        const int slot = t - first_tile(g);
        const float *part = partial + (g * sk.slots + slot) * 32 * kDPartCols + m * kDPartCols;
        v0[u] = part[cl];
        v1[u] = EPI == Epi::SWIGLU ? part[64 + cl] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kReduceBatch; ++u) {
        if (g0 + (int64_t)u * Q > g_hi) break;
        if (g0 + u == g_lo) {
          s0 = v0[u];
          s1 = v1[u];
        } else {
          s0 += v0[u];
          if constexpr (EPI == Epi::SWIGLU) s1 += v1[u];
        }
      }
    }
  }
  if constexpr (Q == 4) {   // every lane (no divergence around the exchanges)
    s0 += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                        0, __builtin_bit_cast(int, s0), 0xB1, 0xF, 0xF, false));
    s0 += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                        0, __builtin_bit_cast(int, s0), 0x4E, 0xF, 0xF, false));
  }
  if (valid && q == 0) {
    const float extra = p.extra_scale ? *p.extra_scale : 1.0f;
    const int arow = p.a_rowmap ? pr / p.a_rowdiv : pr;
    const int sh = p.a_shift ? p.a_shift[arow] : 0;
    if constexpr (EPI == Epi::SWIGLU) {
      const float G = __builtin_ldexpf(s0, sh) * (p.b_global[0][0] * extra);
      const float U = __builtin_ldexpf(s1, sh) * (p.b_global[1][0] * extra);
      const uint32_t hb = f32_to_bf16_bits(G / (1.0f + expf(-G)) * U);
      static_cast<uint16_t *>(p.out)[(int64_t)m * p.ldo + n] = (uint16_t)hb;
      amax = __builtin_fabsf(bf16_bits_to_f32(hb));
    } else {
      float v = __builtin_ldexpf(s0, sh) * (p.b_global[0][0] * extra);
      int64_t orow = m;
      bool ok = true;
      if constexpr (EPI == Epi::DOWN) {
        orow = p.sorted_pairs ? p.sorted_pairs[m] : m;
        ok = orow >= 0;
        if (ok) v *= p.pair_weights[orow];
      }
      if (ok) {
        if (p.out_type == OutType::F32)
          static_cast<float *>(p.out)[orow * p.ldo + n] = v;
        else
          static_cast<uint16_t *>(p.out)[orow * p.ldo + n] = (uint16_t)f32_to_bf16_bits(v);
      }
    }
  }
  if constexpr (EPI == Epi::SWIGLU) {
    if (p.amax_slot) {
      amax = wave_max(amax);
      if ((threadIdx.x & 63) == 0 && amax > 0.0f) atomicMax(p.amax_slot, __float_as_uint(amax));
    }
  }
}

StreamSplit dense_split(Epi epi, int64_t N, int64_t K, int64_t M) {
  const int64_t cols = epi == Epi::SWIGLU ? dense_cols<Epi::SWIGLU>() : dense_cols<Epi::LINEAR>();
  StreamSplit s;
  s.nch = (int)(K / kDC);
  s.units = (N + cols - 1) / cols * s.nch;
  const int64_t g = (int64_t)kDCUs * (M <= 16 ? DenseCfg<1>::PER_CU : DenseCfg<2>::PER_CU);
  s.grid = (int)(g < s.units ? g : s.units);
  const int64_t per = (s.units + s.grid - 1) / s.grid;    // most units of a workgroup
  s.slots = (int)((per + s.nch - 1) / s.nch + 1);
  return s;
}

template <int MS>
hipError_t launch_ms(Epi epi, const GemmArgs &a, int M, const StreamSplit &sk, hipStream_t s) {
  const dim3 grid((unsigned)sk.grid), block(64 * kDWaves);
  switch (epi) {
    case Epi::LINEAR:
      if (a.a_bf16) return hipErrorInvalidValue;
      launch_kernel((dense_gemv_kernel<MS, Epi::LINEAR, false>), grid, block, 0, s, a, M, sk,
                    a.partial);
      break;
    case Epi::SWIGLU:
      if (a.a_bf16)
        launch_kernel((dense_gemv_kernel<MS, Epi::SWIGLU, true>), grid, block, 0, s, a, M, sk,
                      a.partial);
      else
        launch_kernel((dense_gemv_kernel<MS, Epi::SWIGLU, false>), grid, block, 0, s, a, M, sk,
                      a.partial);
      break;
    case Epi::DOWN:
      if (a.a_bf16)
        launch_kernel((dense_gemv_kernel<MS, Epi::DOWN, true>), grid, block, 0, s, a, M, sk,
                      a.partial);
      else
        launch_kernel((dense_gemv_kernel<MS, Epi::DOWN, false>), grid, block, 0, s, a, M, sk,
                      a.partial);
      break;
  }
  return hipGetLastError();
}

}  // namespace

bool dense_gemv_supported(int64_t M, int64_t K) {
  return M >= 1 && M <= 32 && K % kDC == 0 && K >= kDC;
}

TilePlan dense_gemv_plan(Epi epi, int64_t N, int64_t K, int64_t M) {
  TilePlan t;
  const StreamSplit s = dense_split(epi, N, K, M);
  t.ksplit = 1;
  t.partial_floats = (size_t)s.grid * s.slots * 32 * kDPartCols;
  return t;
}

hipError_t launch_dense_gemv(Epi epi, const GemmArgs &a, int M, const TilePlan &plan,
                             const int32_t *ids, hipStream_t s) {
  (void)ids;
  if (!dense_gemv_supported(M, a.K)) return hipErrorInvalidValue;
  const StreamSplit sk = dense_split(epi, a.N, a.K, M);
  if (!a.partial || plan.partial_floats < (size_t)sk.grid * sk.slots * 32 * kDPartCols)
    return hipErrorInvalidValue;
  hipError_t e = M <= 16 ? launch_ms<1>(epi, a, M, sk, s) : launch_ms<2>(epi, a, M, sk, s);
  if (e != hipSuccess) return e;
  const dim3 block(256);
  const bool u32 = (uint64_t)(sk.units + 1) * (uint64_t)sk.grid + (uint64_t)sk.units <
                   ((uint64_t)1 << 32);
  auto reduce = [&](auto epi_c, auto u32_c) {
    constexpr Epi E = decltype(epi_c)::value;
    const dim3 grid((unsigned)(((int64_t)M * a.N * reduce_lanes<E>() + 255) / 256));
    launch_kernel((dense_reduce_kernel<E, decltype(u32_c)::value>), grid, block, 0, s, a, M, sk,
                  (const float *)a.partial);
  };
  auto with_u32 = [&](auto epi_c) {
    if (u32)
      reduce(epi_c, std::true_type{});
    else
      reduce(epi_c, std::false_type{});
  };
  switch (epi) {
    case Epi::LINEAR:
      with_u32(std::integral_constant<Epi, Epi::LINEAR>{});
      break;
    case Epi::SWIGLU:
      with_u32(std::integral_constant<Epi, Epi::SWIGLU>{});
      break;
    case Epi::DOWN:
      with_u32(std::integral_constant<Epi, Epi::DOWN>{});
      break;
  }
  return hipGetLastError();
}

}  // namespace nvfp4

// Expert-grouped NVFP4 GEMM with LDS-staged activations (gfx950 MFMA).
//
// The prefill form of the routed-expert FFN: the tokens routed to one expert
// form a block of rows that reuses that expert's weights, up to 512 prompt
// tokens per chunk (Eider page, "Performance"); the W4A4 experts of the
// Flash-Next checkpoint (Qwen3.8-Flash-Next-NVFP4-SSD-Stream model card,
// "What this model is") arrive here as exact fp16 rows of their quantised
// activations.
//
// A work item is (m-block of up to BM = 16*MS expert-sorted rows, tile of
// 64 NW weight rows, K range).  The NW waves (4, or 1 when the tiles are too
// few to fill the GPU and K too short to split) of a workgroup split the weight rows
// (64 each; for the gate/up pair 32 gate and the same 32 up rows) and share
// the activation rows.  Both operands pass through a three-stage LDS ring of
// 64-wide K chunks, filled by direct global-to-LDS loads (no registers), so
// two chunks are in flight while one is multiplied and two workgroups fit
// on a CU.  A wave reads its weight codes from LDS, dequantises them in
// registers (E2M1 -> fp16 by the packed converter, times the E4M3 block
// scale in packed fp16: exact) and issues 4 * MS v_mfma_f32_16x16x32_f16 per
// 32-wide step.  Subtiles of 16 rows beyond the block's row count are
// skipped, so a block of an expert with few tokens costs its weight stream
// and little else.  Scales of four chunks arrive at once (one 16-byte load
// per weight row instead of four 4-byte ones: the loads, not their bytes,
// limit this path, and a 4-byte load costs the L2 a whole line).  128-row
// blocks run one straight-line loop per count of filled subtiles; smaller
// blocks, whose occupancy LDS decides, keep a single scale buffer and a
// compact loop.
//
// K permutation: in a 64-wide chunk lane group g = lane / 16 supplies
// k = 16 g + 8 i .. +8 at step i (0, 1) for both operands, so a lane needs
// one 8-byte unit of codes and one scale byte per weight row and chunk.
//
// Work order is XCD-aware: consecutive workgroup ids land on different XCDs
// (round robin over 8), so the item space is cut into 8 contiguous ranges
// and XCD x walks range x; the weight tiles of one m-block then run next to
// each other on one XCD and share its L2 copy of the activation rows.
// Split K: when the four-wave tiles are too few to fill the GPU (a dense
// MLP's down projection has 20 per m-block), each tile's K range is cut into
// KS parts; the parts write raw fp32 sums to a workspace and a reduce kernel
// adds them in part order and applies the epilogue, so results stay
// deterministic.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace nvfp4 {
namespace {

constexpr int kChunk = 64;             // K per pipeline stage
constexpr int kStages = 3;
constexpr int kSGroup = 4;             // chunks whose scales one load brings
constexpr int kARow = kChunk * 2;      // bytes of one fp16 activation row per chunk
constexpr int kBRow = kChunk / 2;      // code bytes of one weight row per chunk
constexpr int kXcds = 8;
constexpr int kFillGroups = 512;       // four-wave workgroups that keep every CU busy (2 per CU)

template <int MS, int NW>
struct TileCfg {
  static constexpr int BM = MS * 16;
  static constexpr int BROWS = 64 * NW;                 // weight rows per workgroup
  static constexpr int A_BYTES = BM * kARow;
  static constexpr int B_BYTES = BROWS * kBRow;
  // Scales arrive in groups of kSGroup chunks (16 bytes per weight row) in a
  // buffer after the ring.  128-row blocks (the straight-line chunk)
  // double-buffer it.  Smaller blocks, mostly a few rows of many small
  // experts, are bound by latency and gain from more workgroups per CU,
  // which LDS decides: they keep one buffer and copy each lane's bytes of a
  // group into registers at the group's first chunk.
  static constexpr bool BIG = MS == 8;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int SG_BYTES = BROWS * kSGroup * (kChunk / 16);
  static constexpr int SG_BUFS = BIG ? 2 : 1;
  static constexpr int STAGES = kStages;
  static constexpr int LDS_BYTES = STAGES * STAGE + SG_BUFS * SG_BYTES;
  static constexpr int A_LOADS = A_BYTES / 1024 / NW;   // 1 KB direct loads per wave
  static constexpr int LOADS = A_LOADS + 2;             // per lane and chunk (A, codes)
  static_assert(A_BYTES % (1024 * NW) == 0, "activation stage splits over the waves");
};

template <Epi EPI>
constexpr int cols_per_wave() { return EPI == Epi::SWIGLU ? 32 : 64; }

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// s_waitcnt vmcnt(min(n, N)) then s_barrier, for a run-time n (the count is
// an instruction immediate; waiting for fewer outstanding loads is safe)
template <int N>
__device__ __forceinline__ void wait_vm_then_barrier(int n) {
  if constexpr (N > 0) {
    if (n >= N) {
      // (a plain barrier: __syncthreads would also wait for the newest loads)
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
      return;
    }
    wait_vm_then_barrier<N - 1>(n);
  } else {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  }
}

__device__ __forceinline__ int arow_of(const GemmArgs &p, int pos) {
  return p.a_rowmap ? p.a_rowmap[pos] / p.a_rowdiv : pos;
}

// Max over the 16 lanes of each DPP row (rotations by 8, 4, 2, 1).
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false)));
  return v;
}

// Lane n of each 16-lane DPP row, broadcast to the whole row.
template <int N>
__device__ __forceinline__ uint32_t row16_bcast(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x150 + N, 0xF, 0xF, false);
}

// Gate/up epilogue with the h quantisation folded in (a given global g_h):
// h = bf16(silu(G) * U) as in the plain epilogue, then NVFP4 blocks of 16
// consecutive columns.  Column lr of a fragment sits in lane lr of the
// 16-lane DPP row that holds the row, so each block's absolute maximum is a
// row reduction.  A lane holds 8 elements (j, f) per 16-row subtile; in a
// group of two subtiles (16 elements e), lane lr keeps the maximum of element
// lr's block, works out that block's scale and reciprocal (one pair of
// divisions per 16 elements), and each element takes them back by a row
// broadcast.  The scale, the codes
// and the stored fp16 products follow the quantisation kernel's fp32 steps
// (one correctly rounded operation each), so the output is the same.
// Blocks never straddle N (N % 16 == 0) and a block's 16 lanes share its
// row, so everything runs unconditionally and only the stores are
// predicated.
template <int MS>
__device__ __forceinline__ void store_h_quantised(const GemmArgs &p, const f32x4 (&acc)[MS][4],
                                                  int nrows, int pos0, int col0, float gg,
                                                  float gu, int lane) {
#pragma clang fp contract(off)
  const int lr = lane & 15, lg = lane >> 4;
  const int N = p.N;
  const float g = *p.h_quant_g;
  const float six_g = 6.0f * g;
  // groups of 16 elements: subtiles 2q and 2q + 1 (one pass each, so only 16
  // h values are live at a time)
#pragma unroll
  for (int q = 0; q < (MS + 1) / 2; ++q) {
    float x[16];
    float bmax = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int ms = 2 * q + (e >> 3), j = (e >> 1) & 3, f = e & 1;
      if (ms >= MS) break;
      const int r = ms * 16 + 4 * lg + j;
      const int sh = (p.a_shift && r < nrows) ? p.a_shift[arow_of(p, pos0 + r)] : 0;
      const float G = __builtin_ldexpf(acc[ms][f][j], sh) * gg;
      const float U = __builtin_ldexpf(acc[ms][f + 2][j], sh) * gu;
      x[e] = bf16_bits_to_f32(f32_to_bf16_bits(G / (1.0f + expf(-G)) * U));
      const float amax = row16_max(__builtin_fabsf(x[e]));
      if (lr == e) bmax = amax;
    }
    // this lane's block: element lr of the group
    const uint32_t sc = e4m3_rne_sat(bmax / six_g);
    const float denom = e4m3_to_f32(sc) * g;
    const uint32_t inv_bits = __float_as_uint(denom > 0.0f ? 1.0f / denom : 0.0f);
    // row_shl:1 -> lane lr reads lane lr + 1: even lanes pair the scales of
    // elements f = 0 and f = 1 of one row
    const uint32_t next = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sc, 0x101, 0xF, 0xF, false);
    const uint32_t sc_pair = sc | (next << 8);
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const int ms = 2 * q + (e >> 3), j = (e >> 1) & 3;
      if (ms >= MS) break;
      const int r = ms * 16 + 4 * lg + j;
      float inv0, inv1;
      uint32_t scs;
      // (constant lane indices: the loop is unrolled)
      switch (e) {
#define NVFP4_BC(L)                                             \
  case L:                                                       \
    inv0 = __uint_as_float(row16_bcast<L>(inv_bits));           \
    inv1 = __uint_as_float(row16_bcast<L + 1>(inv_bits));       \
    scs = row16_bcast<L>(sc_pair);                              \
    break;
        NVFP4_BC(0) NVFP4_BC(2) NVFP4_BC(4) NVFP4_BC(6)
        NVFP4_BC(8) NVFP4_BC(10) NVFP4_BC(12) default: NVFP4_BC(14)
#undef NVFP4_BC
      }
      uint32_t code = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x[e] * inv0, x[e + 1] * inv1,
                                                               1.0f, 0);
      code &= (inv0 > 0.0f ? 0x0Fu : 0u) | (inv1 > 0.0f ? 0xF0u : 0u);   // zero scale: +0
      const f16x2 v = e2m1x2_to_f16<0>(code) *
                      __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scs, 1.0f, false);
      if (r < nrows && col0 < N) {
        _Float16 *hrow = static_cast<_Float16 *>(p.out) + (int64_t)(pos0 + r) * p.ldo;
        hrow[col0 + lr] = v[0];
        hrow[col0 + 16 + lr] = v[1];
      }
    }
  }
}

template <int MS, int NW, Epi EPI>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void tile_gemm_kernel(const GemmArgs p) {
  using C = TileCfg<MS, NW>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS_BYTES];
  // (the wave index is uniform: in a scalar register, LDS offsets and loop
  // conditions derived from it stay scalar)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int K = p.K, N = p.N;
  constexpr int kCols = cols_per_wave<EPI>();
  const int n_tiles = (N + NW * kCols - 1) / (NW * kCols);
  const int ksplit = p.ksplit > 1 ? p.ksplit : 1;
  const int n_mb =
      __builtin_amdgcn_readfirstlane(p.n_mblocks_dev ? *p.n_mblocks_dev : p.n_mblocks);
  const int n_items = n_mb * n_tiles * ksplit;
  const int per = (n_items + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  const int item = (blockIdx.x % kXcds) * per + slot;
  if (slot >= per || item >= n_items) return;
  const int kz = item % ksplit;
  const int mn = item / ksplit;
  const int mb = mn / n_tiles, nt = mn - mb * n_tiles;

  int e = 0, pos0, nrows;
  if (p.mblocks) {
    const int4 blk = p.mblocks[mb];
    e = blk.x;
    pos0 = blk.y;
    nrows = blk.z;
  } else {
    pos0 = mb * C::BM;
    nrows = (int)(p.dense_rows - pos0 < C::BM ? p.dense_rows - pos0 : C::BM);
  }
  // the block is the same for the whole workgroup: keep it in scalar
  // registers so the subtile tests below are scalar branches
  e = __builtin_amdgcn_readfirstlane(e);
  pos0 = __builtin_amdgcn_readfirstlane(pos0);
  nrows = __builtin_amdgcn_readfirstlane(nrows);
  const int col0 = (nt * NW + wave) * kCols;

  // ---- loader state.  Workgroup-local weight row R = 64 w + 16 f + r is row
  // r of fragment f of wave w (SWIGLU: fragments 2, 3 are the up rows of the
  // gate rows in fragments 0, 1).  Rows past N reread row N - 1.
  auto weight_row = [&](int R, int &mat) {
    const int w = R >> 6, f = (R >> 4) & 3, r = R & 15;
    mat = (EPI == Epi::SWIGLU && f >= 2) ? 1 : 0;
    const int fr = EPI == Epi::SWIGLU ? (f & 1) : f;
    const int row = (nt * NW + w) * kCols + fr * 16 + r;
    return row < N ? row : N - 1;
  };
  // Codes: LDS row R holds 32 bytes as two 16-byte halves, half h at
  // position h ^ ((R >> 3) & 1).  Direct load j of wave w is instruction
  // q = 2 w + j; it fills 1 KB = rows 32 q .. 32 q + 31, lane l writing
  // position l % 2 of row 32 q + l / 2.
  const uint8_t *csrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int q = 2 * wave + j, R = 32 * q + (lane >> 1);
    int mat;
    const int row = weight_row(R, mat);
    const int h = (lane & 1) ^ ((R >> 3) & 1);
    csrc[j] = p.b_codes[mat] + (int64_t)e * p.b_codes_estride + (int64_t)row * (K / 2) + h * 16;
  }
  // Scales: wave w loads rows 64 w .. 64 w + 63, lane l row 64 w + l.  One
  // 16-byte load per row brings the scales of kSGroup chunks (a group; LDS
  // row stride 16); the chunks of a part's last, incomplete group load their
  // 4 bytes each (LDS row stride 4, one BROWS * 4 area per chunk).  Scale
  // traffic is one row-sized request per weight row per group instead of one
  // per chunk, which the load path, not the byte count, makes worth having.
  const uint8_t *ssrc;
  {
    int mat;
    const int row = weight_row(64 * wave + lane, mat);
    ssrc = p.b_scales[mat] + (int64_t)e * p.b_scales_estride + (int64_t)row * (K / 16);
  }
  // Activations: LDS row r holds 128 bytes as eight 16-byte granules, granule
  // c at position c ^ ((r >> 1) & 7); instruction q = wave + NW j fills rows
  // 8 q .. 8 q + 7, lane l writing position l % 8 of row 8 q + l / 8, so it
  // fetches granule (l % 8) ^ ((4 q + l / 16) & 7).  Rows past the block
  // reread row 0 (finite data, results discarded).
  // (a fixed-size array: with a size that depends on the template arguments
  // the host pass of this compiler drops the kernel's launch stub)
  static_assert(C::A_LOADS <= 16, "activation loads per wave");
  int64_t aoff[16];   // element offsets of this lane's activation pieces
  // Only the 16-row subtiles that hold rows are staged: instruction j of
  // this wave (rows 8 (wave + NW j) ..) is issued when those rows lie below
  // rows16, so a block of a few rows does not fetch 64 or 128 rows of
  // padding; a_loads counts this wave's activation loads per chunk.
  const int rows16 = nrows >= C::BM ? C::BM : (nrows + 15) / 16 * 16;
  int a_loads = 0;
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j) a_loads += 8 * (wave + NW * j) < rows16 ? 1 : 0;
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j) {
    const int q = wave + NW * j;
    const int r = 8 * q + (lane >> 3);
    const int rr = r < nrows ? r : 0;
    const int gran = (lane & 7) ^ ((4 * q + (lane >> 4)) & 7);
    aoff[j] = (int64_t)arow_of(p, pos0 + rr) * p.lda + gran * 8;
  }

  f32x4 acc[MS][4];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[ms][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this part's chunk range: parts of whole scale groups where groups apply
  // (the host makes every part non-empty; an empty one would write zeros)
  const int nch = K / kChunk;
  int cps = (nch + ksplit - 1) / ksplit;
  if (K % (kSGroup * kChunk) == 0) cps = (cps + kSGroup - 1) / kSGroup * kSGroup;
  const int c_begin = kz * cps;
  const int c_end = c_begin + cps < nch ? c_begin + cps : nch;
  const int last = c_end - 1;
  // chunks from c_tail on form the incomplete last group.  Group loads need
  // 16-byte aligned scale rows (K % 256 == 0, aligned matrices) and a part
  // that starts on a group boundary of the row; otherwise every chunk loads
  // its own 4 bytes.
  const int64_t s_off = (int64_t)e * p.b_scales_estride;
  const bool grouped =
      K % (kSGroup * kChunk) == 0 && c_begin % kSGroup == 0 &&
      ((reinterpret_cast<uintptr_t>(p.b_scales[0] + s_off) |
        (EPI == Epi::SWIGLU ? reinterpret_cast<uintptr_t>(p.b_scales[1] + s_off) : 0)) & 15) == 0;
  const int c_tail = __builtin_amdgcn_readfirstlane(
      grouped ? c_begin + (c_end - c_begin) / kSGroup * kSGroup : c_begin);
  uint8_t *const sgroups = lds + C::STAGES * C::STAGE;
  // scale loads issued with chunk c: 1 at a group's first chunk and at each
  // chunk of the incomplete group, else 0
  auto scale_loads = [&](int c) {
    return (c >= c_tail || ((c - c_begin) & (kSGroup - 1)) == 0) ? 1 : 0;
  };

  // Issue the loads of chunk c (K is a multiple of 64) into ring slot c % 3,
  // and its scale load if it has one.
  auto load_chunk = [&](int c) {
    uint8_t *st = lds + (c % C::STAGES) * C::STAGE;
    const int k0 = c * kChunk;
#pragma unroll
    for (int j = 0; j < C::A_LOADS; ++j)
      if (8 * (wave + NW * j) < rows16)   // uniform per wave
        __builtin_amdgcn_global_load_lds(p.A + aoff[j] + k0,
                                         (lds_ptr_t)(st + (wave + NW * j) * 1024), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_global_load_lds(csrc[j] + k0 / 2,
                                       (lds_ptr_t)(st + C::A_BYTES + (2 * wave + j) * 1024), 16, 0,
                                       0);
    const int rel = c - c_begin;
    uint8_t *sg = sgroups + (C::SG_BUFS == 2 ? ((rel / kSGroup) & 1) * C::SG_BYTES : 0);
    if (c >= c_tail)
      __builtin_amdgcn_global_load_lds(ssrc + k0 / 16,
                                       (lds_ptr_t)(sg + (rel & (kSGroup - 1)) * C::BROWS * 4 +
                                                   wave * 256),
                                       4, 0, 0);
    else if ((rel & (kSGroup - 1)) == 0)
      __builtin_amdgcn_global_load_lds(ssrc + k0 / 16, (lds_ptr_t)(sg + wave * 1024), 16, 0, 0);
  };

  // One chunk with NSUB (a compile-time count) subtiles holding rows, so the
  // whole chunk is straight-line code.  Order: the weight codes, the scales
  // and step 0's activation fragments are requested together; step 0's
  // weight fragments are dequantised while those reads land; then each
  // subtile's four step-0 MFMAs are followed by the request of its step-1
  // fragment into the same registers, with step 1's dequantisation spread
  // between them, so LDS latency and VALU work overlap the matrix pipe.
  auto compute = [&](int c, auto nsub_c) {
    constexpr int NSUB = decltype(nsub_c)::value;
    const uint8_t *st = lds + (c % C::STAGES) * C::STAGE;
    const int rel = c - c_begin;
    const uint8_t *sg = sgroups + ((rel / kSGroup) & 1) * C::SG_BYTES;   // (two buffers)
    const bool tail = c >= c_tail;   // uniform
    const int s_row = tail ? 4 : 16;
    const uint8_t *sc = sg + (tail ? (rel & (kSGroup - 1)) * C::BROWS * 4
                                   : (rel & (kSGroup - 1)) * 4) + lg;
    u32x2 w[4];
    uint32_t sb[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int R = 64 * wave + 16 * f + lr;
      const int pos = (((lg >> 1) ^ ((R >> 3) & 1)) << 4) + ((lg & 1) << 3);
      w[f] = *reinterpret_cast<const u32x2 *>(st + C::A_BYTES + R * kBRow + pos);
      sb[f] = sc[R * s_row];
    }
    const uint8_t *abase = st + lr * kARow;
    const int gran0 = ((2 * lg) ^ ((lr >> 1) & 7)) * 16;
    const int gran1 = ((2 * lg + 1) ^ ((lr >> 1) & 7)) * 16;
    f16x8 a[NSUB];
#pragma unroll
    for (int ms = 0; ms < NSUB; ++ms)
      a[ms] = *reinterpret_cast<const f16x8 *>(abase + ms * 16 * kARow + gran0);
    // (scheduling fences keep this order: the compiler otherwise sinks each
    // fragment read next to its MFMAs and waits on it there)
    if constexpr (NSUB >= 4) __builtin_amdgcn_sched_barrier(0);
    f16x2 s2[4];
    f16x8 b0[4], b1[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      f16x2 unused;
      e4m3x2_to_f16_pairs(sb[f], s2[f], unused);
      b0[f] = dequant8_f16(w[f][0], s2[f]);
    }
    if constexpr (NSUB >= 4) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ms = 0; ms < NSUB; ++ms) {
#pragma unroll
      for (int f = 0; f < 4; ++f)
        acc[ms][f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[ms], b0[f], acc[ms][f], 0, 0, 0);
      a[ms] = *reinterpret_cast<const f16x8 *>(abase + ms * 16 * kARow + gran1);
      if (ms < 4) b1[ms] = dequant8_f16(w[ms][1], s2[ms]);
      if constexpr (NSUB >= 4) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int f = NSUB; f < 4; ++f) b1[f] = dequant8_f16(w[f][1], s2[f]);
    if constexpr (NSUB >= 4) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ms = 0; ms < NSUB; ++ms) {
#pragma unroll
      for (int f = 0; f < 4; ++f)
        acc[ms][f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[ms], b1[f], acc[ms][f], 0, 0, 0);
    }
  };

  // The compact chunk for smaller blocks: subtiles past the block's rows are
  // skipped by uniform branches (FULL: all hold rows).
  // Scale bytes of the current group for the compact chunk: byte c' of
  // gbytes[f] is this lane's scale (block lg) of fragment f's row in the
  // group's chunk c'.  They are read from the one group buffer at the
  // group's first chunk, before the loads of the next group (issued two
  // chunks later, after two barriers) overwrite it.
  uint32_t gbytes[4] = {0u, 0u, 0u, 0u};
  auto compute_small = [&](int c, auto full) {
    constexpr bool FULL = decltype(full)::value;
    const uint8_t *st = lds + (c % C::STAGES) * C::STAGE;
    const int rel = c - c_begin, cg = rel & (kSGroup - 1);
    const bool tail = c >= c_tail;   // uniform
    if (!tail && cg == 0) {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int R = 64 * wave + 16 * f + lr;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(sgroups + R * 16);
        // byte lg of each chunk's word: selector lg, lg + 4 picks from
        // (hi, lo) = (word 1, word 0), then the two halves are joined
        const uint32_t sel = 0x0c0c0400u + (uint32_t)lg * 0x0101u;
        const uint32_t lo = __builtin_amdgcn_perm(v[1], v[0], sel);
        const uint32_t hi = __builtin_amdgcn_perm(v[3], v[2], sel);
        gbytes[f] = lo | (hi << 16);
      }
    }
    f16x8 bf[2][4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int R = 64 * wave + 16 * f + lr;
      const int pos = (((lg >> 1) ^ ((R >> 3) & 1)) << 4) + ((lg & 1) << 3);
      const u32x2 w = *reinterpret_cast<const u32x2 *>(st + C::A_BYTES + R * kBRow + pos);
      const uint32_t sbyte = tail ? sgroups[cg * C::BROWS * 4 + R * 4 + lg]
                                  : (gbytes[f] >> (8 * cg)) & 0xffu;
      f16x2 s0, s1;
      e4m3x2_to_f16_pairs(sbyte, s0, s1);
      bf[0][f] = dequant8_f16(w[0], s0);
      bf[1][f] = dequant8_f16(w[1], s0);
    }
    const uint8_t *abase = st + lr * kARow;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int gran = ((2 * lg + i) ^ ((lr >> 1) & 7)) * 16;
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        if (!FULL && ms * 16 >= nrows) break;   // uniform: skip empty subtiles
        const f16x8 a = *reinterpret_cast<const f16x8 *>(abase + ms * 16 * kARow + gran);
#pragma unroll
        for (int f = 0; f < 4; ++f)
          acc[ms][f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bf[i][f], acc[ms][f], 0, 0, 0);
      }
    }
  };

  // Ring of S stages: chunks c + 1 .. c + S - 1 are in flight while chunk c
  // is multiplied.  The wait before each barrier leaves only the loads of
  // chunks c + 1 .. c + S - 2 outstanding (their count depends on which bring
  // scales, and shrinks past the end); the barrier then also guarantees every
  // wave is done with the ring slot and the scale buffer the next loads
  // overwrite (a scale buffer is reused two groups later: S <= 5).
  auto run = [&](auto step) {
    constexpr int S = C::STAGES;
#pragma unroll
    for (int d = 0; d < S - 1; ++d)
      if (c_begin + d <= last) load_chunk(c_begin + d);
    for (int c = c_begin; c <= last; ++c) {
      // loads still allowed in flight: those of chunks c + 1 .. c + S - 2
      int n = 0;
#pragma unroll
      for (int d = 1; d <= S - 2; ++d)
        if (c + d <= last) n += a_loads + 2 + scale_loads(c + d);
      wait_vm_then_barrier<(S - 2) * (C::LOADS + 1)>(n);
      if (c + S - 1 <= last) load_chunk(c + S - 1);
      step(c);
    }
  };
  if (c_begin > last) {
  } else if constexpr (C::BIG) {
    // subtiles holding rows (uniform): one straight-line loop per count
    const int nsub = nrows >= C::BM ? MS : (nrows + 15) / 16;
    auto pick = [&](auto self, auto n) {
      constexpr int NS = decltype(n)::value;
      if constexpr (NS >= 1) {
        if (nsub == NS)
          run([&](int c) { compute(c, std::integral_constant<int, NS>{}); });
        else
          self(self, std::integral_constant<int, NS - 1>{});
      }
    };
    pick(pick, std::integral_constant<int, MS>{});
  } else if (nrows >= C::BM) {
    run([&](int c) { compute_small(c, std::true_type{}); });
  } else {
    run([&](int c) { compute_small(c, std::false_type{}); });
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: lane holds rows 4*lg + j (j = 0..3) of each subtile and
  //      column lr of each fragment.
  if (ksplit > 1) {   // raw sums of this K part -> partial[kz][pos][col]
    const int ncols = EPI == Epi::SWIGLU ? 2 * N : N;
    float *part = p.partial + (int64_t)kz * p.partial_rows * ncols;
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = ms * 16 + 4 * lg + j;
        if (r >= nrows) continue;
        float *prow = part + (int64_t)(pos0 + r) * ncols;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int fr = EPI == Epi::SWIGLU ? (f & 1) : f;
          const int col = col0 + fr * 16 + lr;
          if (col >= N) continue;
          prow[(EPI == Epi::SWIGLU && f >= 2 ? N : 0) + col] = acc[ms][f][j];
        }
      }
    }
    return;
  }
  const float extra = p.extra_scale ? *p.extra_scale : 1.0f;
  if constexpr (EPI == Epi::SWIGLU) {
    const float gg = p.b_global[0][e] * extra, gu = p.b_global[1][e] * extra;
    if (p.h_quant_g) {   // uniform
      store_h_quantised<MS>(p, acc, nrows, pos0, col0, gg, gu, lane);
      return;
    }
    float amax = 0.0f;
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = ms * 16 + 4 * lg + j;
        if (r >= nrows) continue;
        const int pos = pos0 + r;
        const int sh = p.a_shift ? p.a_shift[arow_of(p, pos)] : 0;
        uint16_t *hrow = static_cast<uint16_t *>(p.out) + (int64_t)pos * p.ldo;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int col = col0 + f * 16 + lr;
          if (col >= N) continue;
          const float G = __builtin_ldexpf(acc[ms][f][j], sh) * gg;
          const float U = __builtin_ldexpf(acc[ms][f + 2][j], sh) * gu;
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
    const float gw = p.b_global[0][e] * extra;
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = ms * 16 + 4 * lg + j;
        if (r >= nrows) continue;
        const int pos = pos0 + r;
        const int sh = p.a_shift ? p.a_shift[arow_of(p, pos)] : 0;
        int64_t orow = pos;
        float w = 1.0f;
        if constexpr (EPI == Epi::DOWN) {
          const int pair = p.sorted_pairs[pos];
          orow = pair;
          w = p.pair_weights[pair];
        }
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int col = col0 + f * 16 + lr;
          if (col >= N) continue;
          float v = __builtin_ldexpf(acc[ms][f][j], sh) * gw;
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

// Split-K reduce: element (pos, col) of the output adds the parts' raw sums
// in part order, then applies the same epilogue as the tile kernel.  Row pos
// belongs to expert ids[sorted_pairs[pos]] (expert 0 when ids is null).
template <Epi EPI>
__global__ __launch_bounds__(256) void split_reduce_kernel(const GemmArgs p, int rows,
                                                           const int32_t *ids) {
  const int N = p.N;
  const int ncols = EPI == Epi::SWIGLU ? 2 * N : N;
  const int64_t total = (int64_t)rows * N;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float amax = 0.0f;
  // (positions past the kept pairs hold pair -1: nothing to write)
  if (idx < total && (!p.sorted_pairs || p.sorted_pairs[idx / N] >= 0)) {
    const int pos = (int)(idx / N), col = (int)(idx - (int64_t)pos * N);
    const int e = ids ? ids[p.sorted_pairs[pos]] : 0;
    const float extra = p.extra_scale ? *p.extra_scale : 1.0f;
    const int sh = p.a_shift ? p.a_shift[arow_of(p, pos)] : 0;
    const int64_t stride = (int64_t)p.partial_rows * ncols;
    const float *src = p.partial + (int64_t)pos * ncols + col;
    float g = src[0], u = 0.0f;
    if constexpr (EPI == Epi::SWIGLU) u = src[N];
    for (int kz = 1; kz < p.ksplit; ++kz) {
      g += src[kz * stride];
      if constexpr (EPI == Epi::SWIGLU) u += src[kz * stride + N];
    }
    if constexpr (EPI == Epi::SWIGLU) {
      const float G = __builtin_ldexpf(g, sh) * (p.b_global[0][e] * extra);
      const float U = __builtin_ldexpf(u, sh) * (p.b_global[1][e] * extra);
      const uint32_t hb = f32_to_bf16_bits(G / (1.0f + expf(-G)) * U);
      static_cast<uint16_t *>(p.out)[(int64_t)pos * p.ldo + col] = (uint16_t)hb;
      amax = __builtin_fabsf(bf16_bits_to_f32(hb));
    } else {
      float v = __builtin_ldexpf(g, sh) * (p.b_global[0][e] * extra);
      int64_t orow = pos;
      if constexpr (EPI == Epi::DOWN) {
        orow = p.sorted_pairs[pos];
        v *= p.pair_weights[orow];
      }
      if (p.out_type == OutType::F32)
        static_cast<float *>(p.out)[orow * p.ldo + col] = v;
      else
        static_cast<uint16_t *>(p.out)[orow * p.ldo + col] = (uint16_t)f32_to_bf16_bits(v);
    }
  }
  if constexpr (EPI == Epi::SWIGLU) {
    if (p.amax_slot) {
      amax = wave_max(amax);
      if ((threadIdx.x & 63) == 0 && amax > 0.0f) atomicMax(p.amax_slot, __float_as_uint(amax));
    }
  }
}

template <int MS, int NW>
hipError_t launch_ms(Epi epi, const GemmArgs &a, int ksplit, hipStream_t s) {
  const int cols = NW * (epi == Epi::SWIGLU ? cols_per_wave<Epi::SWIGLU>()
                                            : cols_per_wave<Epi::LINEAR>());
  const int64_t n_tiles = (a.N + cols - 1) / cols;
  int64_t items = n_tiles * (int64_t)a.n_mblocks * ksplit;
  items = (items + kXcds - 1) / kXcds * kXcds;
  if (items < kXcds) items = kXcds;
  GemmArgs g = a;
  g.ksplit = ksplit;
  const dim3 grid((unsigned)items), block(64 * NW);
  switch (epi) {
    case Epi::LINEAR:
      launch_kernel((tile_gemm_kernel<MS, NW, Epi::LINEAR>), grid, block, 0, s, g);
      break;
    case Epi::SWIGLU:
      launch_kernel((tile_gemm_kernel<MS, NW, Epi::SWIGLU>), grid, block, 0, s, g);
      break;
    case Epi::DOWN:
      launch_kernel((tile_gemm_kernel<MS, NW, Epi::DOWN>), grid, block, 0, s, g);
      break;
  }
  return hipGetLastError();
}

template <int NW>
hipError_t launch_nw(Epi epi, const GemmArgs &a, int bm, int ksplit, hipStream_t s) {
  switch (bm) {
    case 16:
    case 32: return launch_ms<2, NW>(epi, a, ksplit, s);
    case 64: return launch_ms<4, NW>(epi, a, ksplit, s);
    default: return launch_ms<8, NW>(epi, a, ksplit, s);
  }
}

}  // namespace

bool tile_gemm_supported(int K) { return K % kChunk == 0; }

TilePlan tile_gemm_plan(Epi epi, int64_t N, int64_t K, int64_t n_mblocks_bound, int64_t rows) {
  TilePlan t;
  const int64_t cols = epi == Epi::SWIGLU ? cols_per_wave<Epi::SWIGLU>()
                                          : cols_per_wave<Epi::LINEAR>();
  const int64_t items4 = n_mblocks_bound * ((N + 4 * cols - 1) / (4 * cols));
  if (items4 >= kFillGroups) return t;                      // four-wave tiles fill the GPU
  const int64_t nch = K / kChunk;
  {
    // too few tiles to fill the GPU: four-wave tiles (each activation stage
    // shared by 256 weight rows) with K split until they fill it; measured
    // faster than one-wave tiles at every dense MLP size (M = 8 to 2048)
    int64_t ks = (kFillGroups + items4 - 1) / items4;
    if (ks > nch / 2) ks = nch / 2;
    if (ks >= 2) {
      // (the kernel rounds a part up to whole scale groups when K % 256 == 0)
      int64_t cps = (nch + ks - 1) / ks;
      if (K % (kSGroup * kChunk) == 0) cps = (cps + kSGroup - 1) / kSGroup * kSGroup;
      t.ksplit = (int)((nch + cps - 1) / cps);
      t.partial_floats = (size_t)t.ksplit * rows * (epi == Epi::SWIGLU ? 2 * N : N);
      return t;
    }
  }
  // K too short to split (under four chunks): one-wave tiles, four times as
  // many items
  t.waves = 1;
  return t;
}

hipError_t launch_tile_gemm(Epi epi, const GemmArgs &a, int bm, const TilePlan &plan,
                            const int32_t *ids, int rows, hipStream_t s) {
  if (!tile_gemm_supported(a.K)) return hipErrorInvalidValue;
  if (plan.ksplit > 1 && (!a.partial || a.partial_rows < rows)) return hipErrorInvalidValue;
  hipError_t err = plan.waves == 4 ? launch_nw<4>(epi, a, bm, plan.ksplit, s)
                                   : launch_nw<1>(epi, a, bm, plan.ksplit, s);
  if (err != hipSuccess || plan.ksplit <= 1) return err;
  GemmArgs g = a;
  g.ksplit = plan.ksplit;
  return launch_split_reduce(epi, g, rows, ids, s);
}

hipError_t launch_split_reduce(Epi epi, const GemmArgs &g, int rows, const int32_t *ids,
                               hipStream_t s) {
  const dim3 grid((unsigned)(((int64_t)rows * g.N + 255) / 256)), block(256);
  switch (epi) {
    case Epi::LINEAR:
      launch_kernel(split_reduce_kernel<Epi::LINEAR>, grid, block, 0, s, g, rows, ids);
      break;
    case Epi::SWIGLU:
      launch_kernel(split_reduce_kernel<Epi::SWIGLU>, grid, block, 0, s, g, rows, ids);
      break;
    case Epi::DOWN:
      launch_kernel(split_reduce_kernel<Epi::DOWN>, grid, block, 0, s, g, rows, ids);
      break;
  }
  return hipGetLastError();
}

}  // namespace nvfp4

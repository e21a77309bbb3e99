// Expert paging: a device pool of S expert slots in front of all E experts'
// NVFP4 weights in pinned host memory (selected experts resident, the rest
// paged in: Eider page, "Why Eider exists").  The plan runs on the device so
// a step never waits for the host: one workgroup marks the experts the step
// needs, keeps the resident ones, gives each missing one a free slot (in slot
// order from a clock hand; a slot is free when it is empty, or holds an expert
// the step does not need whose stamp is older than the step still in flight)
// and remaps the routing ids to slots.  The fetch kernel then reads the
// missing experts' pages straight from host memory into their slots (the
// host does not know how many there are; the kernel reads the count).
#include "common.h"
#include "kernels.h"

namespace nvfp4 {
namespace {

constexpr int kPlanThreads = 1024;   // one thread per expert and per slot (E, S <= 1024)

// Exclusive prefix sum of one flag per thread over the workgroup (1024
// threads); also returns the total.
__device__ int block_exclusive_scan(int v, int &total) {
  __shared__ int wave_sum[kPlanThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  int base = 0;
  total = 0;
  for (int w = 0; w < kPlanThreads / 64; ++w) {
    if (w < wave) base += wave_sum[w];
    total += wave_sum[w];
  }
  __syncthreads();
  return base + incl - v;
}

__global__ __launch_bounds__(256) void cache_init_kernel(int32_t *slot_of, int E,
                                                          int32_t *expert_of, uint32_t *last_use,
                                                          int32_t *hand, int S) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < E) slot_of[i] = -1;
  if (i < S) {
    expert_of[i] = -1;
    last_use[i] = 0u;
  }
  if (i == 0) *hand = 0;
}

__global__ __launch_bounds__(kPlanThreads) void cache_plan_kernel(
    const int32_t *ids, int P, int E, int S, int32_t *slot_of, int32_t *expert_of,
    uint32_t *last_use, int32_t *hand, uint32_t step, uint32_t protect_from, int max_fetch,
    int32_t *slot_ids, int32_t *fetch, int32_t *n_fetch) {
  __shared__ uint8_t need[kPlanThreads];
  __shared__ int32_t miss_list[kPlanThreads];
  __shared__ int32_t victim_list[kPlanThreads];
  const int tid = threadIdx.x;
  need[tid] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += kPlanThreads) {
    const int e = ids[p];
    if ((unsigned)e < (unsigned)E) need[e] = 1;   // (ids outside 0..E-1 are ignored)
  }
  __syncthreads();

  // needed experts: the resident ones are stamped, the missing ones listed in
  // ascending expert order (state entries out of range count as empty, so a
  // damaged state never leads outside the arrays)
  int is_miss = 0;
  if (tid < E && need[tid]) {
    const int s = slot_of[tid];
    if ((unsigned)s < (unsigned)S)
      last_use[s] = step;
    else
      is_miss = 1;
  }
  int n_miss;
  const int mrank = block_exclusive_scan(is_miss, n_miss);
  if (is_miss) miss_list[mrank] = tid;

  // free slots, in slot order starting at the hand (rotated index r)
  int h = *hand;
  if ((unsigned)h >= (unsigned)S) h = 0;
  int is_free = 0, slot = -1;
  if (tid < S) {
    slot = h + tid < S ? h + tid : h + tid - S;
    const int e = expert_of[slot];
    is_free = (unsigned)e >= (unsigned)E || (!need[e] && last_use[slot] < protect_from);
  }
  int n_free;
  const int frank = block_exclusive_scan(is_free, n_free);
  if (is_free) victim_list[frank] = slot;
  __syncthreads();

  // not enough free slots (or more misses than the fetch will copy): nothing
  // moves, *n_fetch = -1, and the missing experts' pairs get slot -1, which
  // every later call drops (the FFN gives them no contribution)
  const bool fits = n_miss <= n_free && n_miss <= max_fetch;
  // missing expert i takes free slot i
  if (fits && tid < n_miss) {
    const int e = miss_list[tid], s = victim_list[tid];
    const int old = expert_of[s];
    if ((unsigned)old < (unsigned)E) slot_of[old] = -1;
    slot_of[e] = s;
    expert_of[s] = e;
    last_use[s] = step;
    fetch[2 * tid] = e;
    fetch[2 * tid + 1] = s;
  }
  if (tid == 0) {
    *n_fetch = fits ? n_miss : -1;
    if (fits && n_miss > 0) {
      const int last = victim_list[n_miss - 1];
      *hand = last + 1 < S ? last + 1 : 0;
    }
  }
  __syncthreads();   // (the slot map writes above are visible to the workgroup)
  for (int p = tid; p < P; p += kPlanThreads) {
    const int e = ids[p];
    const int s = (unsigned)e < (unsigned)E ? slot_of[e] : -1;
    slot_ids[p] = (unsigned)s < (unsigned)S ? s : -1;   // (ids outside 0..E-1, or a failed plan: -1)
  }
}

// One expert's bytes as segments: gate, up, down codes; gate, up, down
// scales (16-byte pieces); then the three 4-byte globals.
struct FetchArgs {
  const uint8_t *src[9];
  uint8_t *dst[9];
  int64_t bytes[9];
};

// A fixed grid strides over the pieces of one fetched expert after another
// (no barrier between experts: a wave moves on as soon as its pieces are
// done), four pieces' loads in flight per thread, so that many host reads
// are outstanding on the link at once.  With nothing to fetch every
// workgroup leaves after one read.
__global__ __launch_bounds__(256) void cache_fetch_kernel(const FetchArgs a, const int32_t *fetch,
                                                           const int32_t *n_fetch, int max_fetch) {
  const int n = min(*n_fetch, max_fetch);
  const int64_t gtid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t gstride = (int64_t)gridDim.x * 256;
  for (int i = 0; i < n; ++i) {
    const int e = fetch[2 * i], s = fetch[2 * i + 1];
#pragma unroll 1
    for (int j = 0; j < 6; ++j) {
      const u32x4 *src = reinterpret_cast<const u32x4 *>(a.src[j] + (int64_t)e * a.bytes[j]);
      u32x4 *dst = reinterpret_cast<u32x4 *>(a.dst[j] + (int64_t)s * a.bytes[j]);
      const int64_t n16 = a.bytes[j] / 16;
      int64_t q = gtid;
      for (; q + 3 * gstride < n16; q += 4 * gstride) {
        const u32x4 v0 = src[q], v1 = src[q + gstride], v2 = src[q + 2 * gstride],
                    v3 = src[q + 3 * gstride];
        dst[q] = v0;
        dst[q + gstride] = v1;
        dst[q + 2 * gstride] = v2;
        dst[q + 3 * gstride] = v3;
      }
      for (; q < n16; q += gstride) dst[q] = src[q];
    }
    if (gtid < 3) {   // the globals
      const int j = 6 + (int)gtid;
      *reinterpret_cast<float *>(a.dst[j] + (int64_t)s * 4) =
          *reinterpret_cast<const float *>(a.src[j] + (int64_t)e * 4);
    }
  }
}

}  // namespace

hipError_t launch_cache_init(int32_t *slot_of, int E, int32_t *expert_of, uint32_t *last_use,
                             int32_t *hand, int S, hipStream_t s) {
  const int n = E > S ? E : S;
  launch_kernel(cache_init_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, slot_of, E,
                expert_of, last_use, hand, S);
  return hipGetLastError();
}

hipError_t launch_cache_plan(const int32_t *ids, int P, int E, int S, int32_t *slot_of,
                             int32_t *expert_of, uint32_t *last_use, int32_t *hand, uint32_t step,
                             uint32_t protect_from, int max_fetch, int32_t *slot_ids,
                             int32_t *fetch, int32_t *n_fetch, hipStream_t s) {
  if (E > kPlanThreads || S > kPlanThreads) return hipErrorInvalidValue;
  launch_kernel(cache_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, ids, P, E, S, slot_of,
                expert_of, last_use, hand, step, protect_from, max_fetch, slot_ids, fetch,
                n_fetch);
  return hipGetLastError();
}

hipError_t launch_cache_fetch(const ExpertPtrs &host, const ExpertPtrs &pool, int64_t H,
                              int64_t I, const int32_t *fetch, const int32_t *n_fetch,
                              int max_fetch, hipStream_t s) {
  if (max_fetch <= 0) return hipSuccess;
  const int64_t gu_codes = I * (H / 2), gu_scales = I * (H / 16);
  const int64_t d_codes = H * (I / 2), d_scales = H * (I / 16);
  FetchArgs a;
  const int64_t bytes[9] = {gu_codes, gu_codes, d_codes, gu_scales, gu_scales, d_scales, 4, 4, 4};
  for (int j = 0; j < 9; ++j) {
    a.src[j] = host.p[j];
    a.dst[j] = const_cast<uint8_t *>(pool.p[j]);
    a.bytes[j] = bytes[j];
    if (j < 6 && bytes[j] % 16 != 0) return hipErrorInvalidValue;
  }
  // enough workgroups for one expert's codes in a few passes, at most 1024
  int64_t wg = (gu_codes / 16 + 4 * 256 - 1) / (4 * 256);
  if (wg > 1024) wg = 1024;
  if (wg < 1) wg = 1;
  launch_kernel(cache_fetch_kernel, dim3((unsigned)wg), dim3(256), 0, s, a, fetch, n_fetch,
                max_fetch);
  return hipGetLastError();
}

}  // namespace nvfp4

// The quota controller on the device: before the backward pass, from the
// number of pairs routed to each expert and one budget of pairs this GPU may
// carry (the memory and network limits), the per-expert quotas for the whole
// layer call (LRMoE page 1, section on what LRMoE does, bullet "Квоты до
// вычислений"; page 2, bullet "Des quotas avant le calcul").  The pages give
// no formula; the rule is water-filling caps that trim the most loaded experts
// first (the same rule as the host controller lrm_quota_waterfill):
//   tau = the largest integer with sum_e min(n_e, tau) <= budget;
//   q_e = min(n_e, tau), plus one for the first budget - sum_e min(n_e, tau)
//         experts (lowest index) with n_e > tau;  q = n when budget >= sum n.
// One 1024-thread block: the counts (read, or summed from the bucketing
// histogram of the pairs) in registers, tau by bisection with block sums, the
// leftover pairs handed out by a block scan of the cut experts.  Integer
// arithmetic only: the result is exact and equal to the host controller's.
#include "common.h"
#include "launch.h"

namespace lrm {

constexpr int kQThreads = 1024;
constexpr int kQPer = 4;  // experts per thread (E <= kQThreads * kQPer)

__device__ __forceinline__ int64_t block_sum64(int64_t v, int64_t* lds) {
  constexpr int NW = kQThreads / kWave;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  const int w = threadIdx.x >> 6;
  if (lane_id() == 0) lds[w] = v;
  __syncthreads();
  int64_t t = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) t += lds[i];
  __syncthreads();
  return t;
}

__device__ __forceinline__ int block_max(int v, int* lds) {
  constexpr int NW = kQThreads / kWave;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  const int w = threadIdx.x >> 6;
  if (lane_id() == 0) lds[w] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) t = max(t, lds[i]);
  __syncthreads();
  return t;
}

// counts: device [E] (negative entries count as 0), or nullptr: n_e is the
// sum of row e of the bucketing histogram blkcnt [E][nblk] (then the blocks'
// index-error bits blkerr [nblk] go to err[0]; err may be nullptr otherwise).
__global__ __launch_bounds__(kQThreads) void k_quota_waterfill(
    int E, const int32_t* __restrict__ counts, const int32_t* __restrict__ blkcnt, int nblk,
    const uint32_t* __restrict__ blkerr, uint32_t* __restrict__ err, int64_t budget,
    int32_t* __restrict__ quota) {
  __shared__ int64_t lds64[kQThreads / kWave];
  __shared__ int lds[kQThreads / kWave + 1];
  LRM_DYN_SHARED(int, nsh);  // [E]
  if (counts) {
    for (int e = threadIdx.x; e < E; e += kQThreads) nsh[e] = max(counts[e], 0);
  } else {
    // one wave per expert row of the histogram
    const int w = threadIdx.x >> 6, l = lane_id();
    for (int e = w; e < E; e += kQThreads / kWave) {
      const int32_t* row = blkcnt + (int64_t)e * nblk;
      int s = 0;
      for (int b = l; b < nblk; b += kWave) s += row[b];
      s = wave_sum(s);
      if (l == 0) nsh[e] = s;
    }
    if (err) {
      __shared__ uint32_t eor;
      if (threadIdx.x == 0) eor = 0u;
      __syncthreads();
      uint32_t bad = 0u;
      for (int b = threadIdx.x; b < nblk; b += kQThreads) bad |= blkerr[b];
      if (bad) atomicOr(&eor, bad);
      __syncthreads();
      if (threadIdx.x == 0) err[0] = eor;
    }
  }
  __syncthreads();
  // this thread's experts: a contiguous run, so that the scan below hands the
  // leftover pairs out in expert order
  const int e0 = threadIdx.x * kQPer;
  int n[kQPer];
  int64_t local = 0;
  int nmax = 0;
#pragma unroll
  for (int j = 0; j < kQPer; ++j) {
    n[j] = e0 + j < E ? nsh[e0 + j] : 0;
    local += n[j];
    nmax = max(nmax, n[j]);
  }
  const int64_t total = block_sum64(local, lds64);
  if (budget >= total) {
#pragma unroll
    for (int j = 0; j < kQPer; ++j)
      if (e0 + j < E) quota[e0 + j] = n[j];
    return;
  }
  // S(tau) = sum_e min(n_e, tau) is non-decreasing; S(0) = 0 <= budget < S(max n)
  int lo = 0, hi = block_max(nmax, lds);
  int64_t s_lo = 0;
  while (hi - lo > 1) {  // invariant: S(lo) <= budget < S(hi)
    const int mid = lo + (hi - lo) / 2;
    int64_t part = 0;
#pragma unroll
    for (int j = 0; j < kQPer; ++j) part += min(n[j], mid);
    const int64_t s = block_sum64(part, lds64);
    if (s <= budget) {
      lo = mid;
      s_lo = s;
    } else {
      hi = mid;
    }
  }
  const int tau = lo;
  const int64_t left = budget - s_lo;  // < the number of experts above tau
  int cut = 0;
#pragma unroll
  for (int j = 0; j < kQPer; ++j) cut += n[j] > tau ? 1 : 0;
  int tot;
  int rank = block_excl_scan<kQThreads>(cut, lds, &tot);
#pragma unroll
  for (int j = 0; j < kQPer; ++j) {
    if (e0 + j >= E) continue;
    int q = min(n[j], tau);
    if (n[j] > tau) {
      if (rank < left) ++q;
      ++rank;
    }
    quota[e0 + j] = q;
  }
}

hipError_t launch_quota_waterfill(const QuotaArgs& a, hipStream_t s) {
  if (a.E < 1 || a.E > kQThreads * kQPer || !a.quota || a.budget < 0) return hipErrorInvalidValue;
  if (!a.counts) {
    // the per-expert counts of the pairs, from the bucketing histogram
    if (a.N > 0 && (!a.token || !a.expert)) return hipErrorInvalidValue;
    const int nblk = bucket_blocks(a.N);
    const hipError_t e =
        launch_bucket_count(a.N, a.T, a.E, a.token, a.expert, a.blkcnt, a.blkerr, nullptr, s);
    if (e != hipSuccess) return e;
    // (no pairs: every count is 0 and the error word is cleared)
    LRM_LAUNCH(1, kQThreads, a.E * sizeof(int), s, k_quota_waterfill)(
        a.E, nullptr, a.blkcnt, a.N > 0 ? nblk : 0, a.blkerr, a.err, a.budget, a.quota);
  } else {
    LRM_LAUNCH(1, kQThreads, a.E * sizeof(int), s, k_quota_waterfill)(
        a.E, a.counts, nullptr, 0, nullptr, nullptr, a.budget, a.quota);
  }
  return hipGetLastError();
}

}  // namespace lrm

// Per-expert top-quota selection and packed-row assignment.
//
// A controller fixes one quota per expert for the layer call; when the
// gradient arrives, each expert keeps its highest-scoring pairs within the
// quota (LRMoE page 1, bullets "Квоты до вычислений" and "Отбор по метрике
// LRM").  Kept rows are then packed expert by expert with no padding (bullet
// "Физическое уплотнение").  Ties in score go to the lower pair index.
//
// Steps (all deterministic, no floating-point atomics, no host sync):
//   1. bucket_count   per-chunk expert histograms (validates indices)
//   2. bucket_scan    candidate offsets per expert and kept offsets
//                     M_e = min(q_e, n_e), both exclusive prefix sums
//   3. bucket_scatter stable counting-sort scatter of pair ids (ascending
//                     inside an expert) and their fp32 score bits
//   4. select         one workgroup per expert: 4-pass 8-bit radix search for
//                     the M_e-th largest key, then a block prefix scan in
//                     candidate order that keeps keys above the threshold and
//                     the first (lowest-index) ties, and writes packed rows.
// Scores are >= 0, so their fp32 bit patterns order like the values.
#include <cstdlib>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace lrm {

constexpr int kSelThreads = 1024;
constexpr int kSelRegKeys = 8;  // keys per thread held in registers by k_select
constexpr int kSelRunKeys = 8;  // keys per thread and round of k_select's keep pass (larger experts)
static_assert(kSelRunKeys * kSelThreads < (1 << 16), "packed round counts of k_select");
constexpr int kScanTile = 8192;  // block counts staged in LDS per round by k_bucket_scan
constexpr int kScatBatch = 8;   // 64-pair groups per wave loaded ahead by k_bucket_scatter

// Kept offsets out[e] = min(M_0 + ... + M_{e-1}, cap) for e in [0, E] (cap < 0:
// no cap), with M_e in mcount (LDS, E <= 4 * kSelThreads).  When the total
// passes cap (only a captured call replayed with other host quotas than it
// was sized with), every later expert keeps fewer rows, so all kernels after
// it see at most cap packed rows; mcount then holds the capped counts.
// Returns true (in every thread) if the total passed cap.
__device__ bool scan_kept_capped(int E, int* mcount, int32_t* out, int64_t cap, int* lds) {
  constexpr int per = 4;
  const int i0 = threadIdx.x * per;
  int v[per];
  int local = 0;
#pragma unroll
  for (int j = 0; j < per; ++j) {
    v[j] = (i0 + j < E) ? mcount[i0 + j] : 0;
    local += v[j];
  }
  int total;
  int run = block_excl_scan<kSelThreads>(local, lds, &total);
  const int c = cap < 0 ? 0x7fffffff : (int)min<int64_t>(cap, 0x7fffffff);
#pragma unroll
  for (int j = 0; j < per; ++j) {
    if (i0 + j < E) {
      const int lo = min(run, c);
      out[i0 + j] = lo;
      if (total > c) mcount[i0 + j] = min(run + v[j], c) - lo;
    }
    run += v[j];
  }
  if (threadIdx.x == 0) out[E] = min(total, c);
  __syncthreads();  // capped counts visible to the whole block
  return total > c;
}

// tok_off[t] for the tokens t that start at pair p (p in [0, N]): the first
// pair whose token is >= t.
__device__ __forceinline__ void token_offsets_at(int64_t p, int N, int T,
                                                 const int32_t* __restrict__ token,
                                                 int32_t* __restrict__ tok_off) {
  const int lo = (p == 0) ? 0 : min(max(token[p - 1], -1), T - 1) + 1;
  const int hi = (p == N) ? T : min(max(token[p], 0), T);
  for (int t = lo; t <= hi; ++t) tok_off[t] = (int32_t)p;
}

__global__ __launch_bounds__(256) void k_bucket_count(int N, int T, int E, int chunk,
                                                      const int32_t* __restrict__ token,
                                                      const int32_t* __restrict__ expert,
                                                      int32_t* __restrict__ blkcnt,
                                                      uint32_t* __restrict__ blkerr,
                                                      int32_t* __restrict__ tok_off) {
  LRM_DYN_SHARED(int, hist);
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t p0 = (int64_t)blockIdx.x * chunk;
  const int64_t p1 = min<int64_t>(p0 + chunk, N);
  uint32_t bad = 0;
  for (int64_t p = p0 + threadIdx.x; p < p1; p += 256) {
    const int e = expert[p];
    const int t = token[p];
    if (e < 0 || e >= E) bad |= kErrExpertRange;
    if (t < 0 || t >= T) bad |= kErrTokenRange;
    if (p > 0 && token[p - 1] > t) bad |= kErrTokenOrder;
    if (e >= 0 && e < E && t >= 0 && t < T) atomicAdd(&hist[e], 1);
    if (tok_off) token_offsets_at(p, N, T, token, tok_off);
  }
  if (tok_off && p1 == N && threadIdx.x == 0) token_offsets_at(N, N, T, token, tok_off);
  // this block's error bits: one word per block, written every call (no
  // zeroing pass); the scan kernel folds them into the call's error word
  __shared__ uint32_t berr;
  if (threadIdx.x == 0) berr = 0u;
  __syncthreads();
  if (bad) atomicOr(&berr, bad);
  __syncthreads();
  if (threadIdx.x == 0) blkerr[blockIdx.x] = berr;
  for (int e = threadIdx.x; e < E; e += 256) blkcnt[(int64_t)e * gridDim.x + blockIdx.x] = hist[e];
}

// Large histograms (E * nblk of at least kRowsMinWork counts, nblk at most
// kRowsMaxBlk): the rows of blkcnt are scanned by many workgroups, one wave
// per expert, before k_bucket_scan (one workgroup) makes the offsets:
// blkcnt[e][b] -> exclusive within-expert offset of block b, and
// cand_off[e] = n_e for k_bucket_scan to take (rows_done).  Each lane loads
// all its counts of the row before the wave scans them.  (On the 65536-token
// workload, E = 128 rows of 1024 blocks, one workgroup took 47 us over the
// rows.)  The CPU-emulation build lowers the bound so its small problems run
// this path.
#ifndef LRM_BUCKET_ROWS_MIN
#define LRM_BUCKET_ROWS_MIN 32768
#endif
constexpr int64_t kRowsMinWork = LRM_BUCKET_ROWS_MIN;
constexpr int kRowsMaxBlk = 1024;
constexpr int kRowsPer = kRowsMaxBlk / kWave;  // counts per lane
__global__ __launch_bounds__(kSelThreads) void k_bucket_rows(int nblk, int E,
                                                             int32_t* __restrict__ blkcnt,
                                                             int32_t* __restrict__ cand_off) {
  const int e = blockIdx.x * (kSelThreads / kWave) + (int)(threadIdx.x >> 6);
  if (e >= E) return;  // whole waves (no barrier in this kernel)
  const int l = lane_id();
  int32_t* row = blkcnt + (int64_t)e * nblk;
  int v[kRowsPer];
#pragma unroll
  for (int u = 0; u < kRowsPer; ++u) {
    const int b = u * kWave + l;
    v[u] = b < nblk ? row[b] : 0;
  }
  int run = 0;
#pragma unroll
  for (int u = 0; u < kRowsPer; ++u) {
    const int b = u * kWave + l;
    const int incl = wave_incl_scan(v[u]);
    if (b < nblk) row[b] = run + incl - v[u];
    run += __shfl(incl, kWave - 1, kWave);
  }
  if (l == 0) cand_off[e] = run;
}

// blkcnt[e][b] -> exclusive within-expert offset of block b (one wave scans
// one expert's block counts, 64 at a time); cand_off = prefix of the
// per-expert counts; offsets = prefix of M_e = min(quota_e, n_e)
// (quota == nullptr: keep all).  rows_done: k_bucket_rows has scanned the
// rows and left n_e in cand_off[e].
// Also: err[0] = OR of the blocks' error bits; mt_off (optional) = prefix of
// ceil(M_e / mt_bm), the dX row tiles of the grouped GEMM.
__global__ __launch_bounds__(kSelThreads) void k_bucket_scan(int nblk, int E,
                                                             int32_t* __restrict__ blkcnt,
                                                             const int32_t* __restrict__ quota,
                                                             int32_t* __restrict__ cand_off,
                                                             int32_t* __restrict__ offsets,
                                                             const uint32_t* __restrict__ blkerr,
                                                             uint32_t* __restrict__ err,
                                                             int32_t* __restrict__ mt_off,
                                                             int mt_bm, QuotaPack qp,
                                                             int use_qp, int64_t max_kept,
                                                             int rows_done) {
  LRM_DYN_SHARED(int, counts);  // [2E]: counts, then kept counts min(quota, count)
  __shared__ int lds[kSelThreads / kWave + 1];
  __shared__ uint32_t eor;
  if (threadIdx.x == 0) eor = 0u;
  // the error words, the quotas and the first round of counts are all
  // requested before any of them is waited for
  uint32_t bad = 0u;
  for (int b = threadIdx.x; b < nblk; b += kSelThreads) bad |= blkerr[b];
  int* mcount = counts + E;
  // quotas: device array, or by value (E <= kQuotaPackMax), or keep all
  auto quota_of = [&](int e) {
    return quota ? max(quota[e], 0) : (use_qp ? max(qp.q[e], 0) : 0x7fffffff);
  };
  const int q0 = threadIdx.x < E ? quota_of(threadIdx.x) : 0;
  const int w = threadIdx.x >> 6, l = lane_id();
  constexpr int NW = kSelThreads / kWave;
  constexpr int PER = kScanTile / kSelThreads;
  // Rounds of R whole rows (rows of consecutive experts are contiguous in
  // blkcnt): the block loads a round's counts with coalesced loads, issued
  // before the previous round is scanned, stages them in LDS, and wave w
  // scans rows w, w + NW, ... of the round from there.
  __shared__ int stage[kScanTile];
  const int R = nblk > 0 ? kScanTile / nblk : E;  // nblk <= kScanTile
  int v[PER];
  auto load_round = [&](int e0) {
    const int cnt = min(R, E - e0) * nblk;
    const int32_t* src = blkcnt + (int64_t)e0 * nblk;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = threadIdx.x + u * kSelThreads;
      v[u] = idx < cnt ? src[idx] : 0;
    }
  };
  if (E > 0 && !rows_done) load_round(0);
  if (threadIdx.x < E) mcount[threadIdx.x] = q0;
  for (int e = threadIdx.x + kSelThreads; e < E; e += kSelThreads) mcount[e] = quota_of(e);
  __syncthreads();  // eor and mcount initialised
  if (bad) atomicOr(&eor, bad);
  if (rows_done) {
    for (int e = threadIdx.x; e < E; e += kSelThreads) {
      const int n = cand_off[e];
      counts[e] = n;
      mcount[e] = min(mcount[e], n);
    }
  }
  for (int e0 = 0; e0 < E && !rows_done; e0 += R) {
    const int rows = min(R, E - e0);
#pragma unroll
    for (int u = 0; u < PER; ++u) stage[threadIdx.x + u * kSelThreads] = v[u];
    __syncthreads();
    if (e0 + R < E) load_round(e0 + R);
    for (int r = w; r < rows; r += NW) {
      int32_t* row = blkcnt + (int64_t)(e0 + r) * nblk;
      int run = 0;
      for (int b0 = 0; b0 < nblk; b0 += kWave) {
        const int b = b0 + l;
        const int x = b < nblk ? stage[r * nblk + b] : 0;
        const int incl = wave_incl_scan(x);
        if (b < nblk) row[b] = run + incl - x;
        run += __shfl(incl, kWave - 1, kWave);
      }
      if (l == 0) {
        counts[e0 + r] = run;
        mcount[e0 + r] = min(mcount[e0 + r], run);
      }
    }
    __syncthreads();
  }
  __syncthreads();
  block_scan_array<kSelThreads>(E, [&](int e) { return counts[e]; }, cand_off, lds);
  const bool over = scan_kept_capped(E, mcount, offsets, max_kept, lds);
  if (mt_off) {
    block_scan_array<kSelThreads>(
        E, [&](int e) { return (mcount[e] + mt_bm - 1) / mt_bm; }, mt_off, lds);
  }
  if (threadIdx.x == 0) err[0] = eor | (over ? kErrCapacity : 0u);
}

// Stage-two offsets: candidates of e are cand_off[e]..cand_off[e+1].
__global__ __launch_bounds__(kSelThreads) void k_kept_offsets(int E,
                                                              const int32_t* __restrict__ cand_off,
                                                              const int32_t* __restrict__ quota,
                                                              int32_t* __restrict__ offsets,
                                                              QuotaPack qp, int use_qp,
                                                              uint32_t* __restrict__ err,
                                                              int64_t cap) {
  __shared__ int lds[kSelThreads / kWave + 1];
  LRM_DYN_SHARED(int, mcount);  // [E]
  for (int e = threadIdx.x; e < E; e += kSelThreads) {
    const int n = cand_off[e + 1] - cand_off[e];
    mcount[e] = quota ? min(max(quota[e], 0), n) : (use_qp ? min(max(qp.q[e], 0), n) : n);
  }
  __syncthreads();
  const bool over = scan_kept_capped(E, mcount, offsets, cap, lds);
  // (the call's error word was written by an earlier kernel of the stream)
  if (threadIdx.x == 0 && over) err[0] |= kErrCapacity;
}

// One wave per chunk; stable scatter in pair order.  Lanes with the same
// expert are matched with ballots over the expert-id bits.
__global__ __launch_bounds__(64) void k_bucket_scatter(int N, int T, int E, int chunk,
                                                       const int32_t* __restrict__ token,
                                                       const int32_t* __restrict__ expert,
                                                       const int32_t* __restrict__ blkcnt,
                                                       const int32_t* __restrict__ cand_off,
                                                       const float* __restrict__ score,
                                                       int32_t* __restrict__ cand,
                                                       uint32_t* __restrict__ keys,
                                                       int32_t* __restrict__ pos, int keep_all) {
  LRM_DYN_SHARED(int, run);  // [E]
  const int l = lane_id();
  const int64_t p0 = (int64_t)blockIdx.x * chunk;
  const int64_t p1 = min<int64_t>(p0 + chunk, N);
  // groups of 64 pairs are taken kScatBatch at a time, their expert, token
  // and score loaded before the first is ranked (the first batch before the
  // running offsets are read)
  int ev[kScatBatch], tv[kScatBatch];
  float sv[kScatBatch];
  auto load_batch = [&](int64_t base0) {
#pragma unroll
    for (int u = 0; u < kScatBatch; ++u) {
      const int64_t p = base0 + u * kWave + l;
      const bool in = p < p1;
      ev[u] = in ? expert[p] : -1;
      tv[u] = in ? token[p] : -1;
      sv[u] = (in && keys) ? score[p] : 0.f;
    }
  };
  load_batch(p0);
  for (int e = l; e < E; e += kWave) run[e] = cand_off[e] + blkcnt[(int64_t)e * gridDim.x + blockIdx.x];
  __syncthreads();
  const int nbits = (E > 1) ? 32 - __clz(E - 1) : 0;
  const uint64_t lt_mask = (l == 0) ? 0ull : (~0ull >> (64 - l));
  for (int64_t base0 = p0; base0 < p1; base0 += kScatBatch * kWave) {
    if (base0 != p0) load_batch(base0);
#pragma unroll
    for (int u = 0; u < kScatBatch; ++u) {
      const int64_t base = base0 + u * kWave;
      if (base >= p1) break;
      const int64_t p = base + l;
      const bool in = p < p1;
      const bool valid = in && ev[u] >= 0 && ev[u] < E && tv[u] >= 0 && tv[u] < T;
      const int e = valid ? ev[u] : 0;
      uint64_t m = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
      }
      const int rank = __popcll(m & lt_mask);
      const int dst = valid ? run[e] + rank : 0;
      // every lane has read its expert's running offset before the group
      // leader advances it (lockstep within the wave)
      __builtin_amdgcn_wave_barrier();
      if (valid) {
        cand[dst] = (int32_t)p;
        if (keys) keys[dst] = __float_as_uint(sv[u]);
        if (keep_all) pos[p] = dst;
        if (rank == 0) run[e] += __popcll(m);
      } else if (in) {
        pos[p] = -1;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// One workgroup per expert.  keys[c] and ids cand[c] (or c itself when cand is
// null) for candidates c in [cand_off[e], cand_off[e+1]), ascending id.
// Candidates and packed slots are clipped to [0, limit), the extent of keys,
// cand, pos and kept (offsets beyond it arise only when a captured call is
// replayed with other host quotas, flagged by the offsets kernels).
//
// The threshold is the m-th largest key, found in three radix passes (bits
// 20-31, 10-19, 0-9).  The 4096 bins of the first digit spread keys that share
// an exponent; with 256 bins a few hot bins serialized the LDS atomics.
// Experts of up to kSelRegKeys * kSelThreads candidates hold their keys in
// registers, thread t the run of K = ceil(n / kSelThreads) consecutive
// candidates from tK; larger ones are read from global memory, strided
// (coalesced) by the passes.  Then, in candidate order, rounds of runs of
// consecutive candidates per thread: each thread counts its keys above the
// threshold and equal to it, one block scan of each count gives it its
// first slot, and it keeps the keys above the threshold and the first r
// equal ones of the expert.  The round's slots are staged in LDS and
// written out by consecutive lanes on consecutive candidates.
//
// select_expert: the workgroup's expert has candidates c0 .. c0 + n - 1 and
// keeps m of them at packed slots o .. o + m - 1 (all clipped already).  Its
// pointers are plain (no restrict): the one-launch selection below writes
// keys and cand earlier in the same kernel.
__device__ __forceinline__ void select_expert(int c0, int n, int o, int m, const uint32_t* keys,
                                              const int32_t* cand, int32_t* pos, int32_t* kept) {
  const int tid = threadIdx.x;
  // the passes' histograms (4096 + 1024 bins), then a round's slots
  constexpr int kHist = kSelRunKeys * kSelThreads > 4096 + 1024 ? kSelRunKeys * kSelThreads
                                                                 : 4096 + 1024;
  __shared__ int hist[kHist];
  __shared__ int lds[kSelThreads / kWave + 1];
  __shared__ uint32_t sh_prefix[2];
  __shared__ int sh_rank[2];
  auto id_of = [&](int c) -> int { return cand ? cand[c] : c; };

  if (m >= n) {
    for (int i = tid; i < n; i += kSelThreads) {
      const int id = id_of(c0 + i);
      kept[o + i] = id;
      pos[id] = o + i;
    }
    return;
  }
  if (m <= 0) {
    for (int i = tid; i < n; i += kSelThreads) pos[id_of(c0 + i)] = -1;
    return;
  }
  const int K = (n + kSelThreads - 1) / kSelThreads;  // run length (uniform)
  const int i0 = tid * K;
  const int cnt = max(0, min(K, n - i0));  // keys of this thread's run
  const bool in_regs = K <= kSelRegKeys;
  uint32_t kr[kSelRegKeys];
#pragma unroll
  for (int j = 0; j < kSelRegKeys; ++j) {
    kr[j] = 0u;
    if (in_regs && j < K) {
      const uint32_t v = keys[c0 + min(i0 + j, n - 1)];
      kr[j] = j < cnt ? v : 0u;
    }
  }
  int* h0 = hist;         // 4096 bins: pass 1, then the first 1024 for pass 3
  int* h1 = hist + 4096;  // 1024 bins: pass 2
  for (int i = tid; i < 4096 + 1024; i += kSelThreads) hist[i] = 0;
  __syncthreads();
  uint32_t prefix = 0, pmask = 0;
  int r = m;
  // One pass: count the keys under the current prefix by digit (shift; nb
  // bins in h), then find the digit of the r-th largest.
  auto pass = [&](int* h, int shift, int nb, int buf) {
    const uint32_t dm = (uint32_t)(nb - 1);
    if (in_regs) {
#pragma unroll
      for (int j = 0; j < kSelRegKeys; ++j)
        if (j < cnt && (kr[j] & pmask) == prefix) atomicAdd(&h[(kr[j] >> shift) & dm], 1);
    } else {
      int i = tid;
      for (; i + 3 * kSelThreads < n; i += 4 * kSelThreads) {
        uint32_t k4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) k4[u] = keys[c0 + i + u * kSelThreads];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if ((k4[u] & pmask) == prefix) atomicAdd(&h[(k4[u] >> shift) & dm], 1);
      }
      for (; i < n; i += kSelThreads) {
        const uint32_t k = keys[c0 + i];
        if ((k & pmask) == prefix) atomicAdd(&h[(k >> shift) & dm], 1);
      }
    }
    __syncthreads();
    // thread t holds the bins nb-1-q*t-i (q = nb / kSelThreads, descending)
    const int q = nb / kSelThreads;
    int c[4];
    int local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = i < q ? h[nb - 1 - q * tid - i] : 0;
      local += c[i];
    }
    int tot;
    int before = block_excl_scan<kSelThreads>(local, lds, &tot);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < q && before < r && before + c[i] >= r) {
        sh_prefix[buf] = prefix | ((uint32_t)(nb - 1 - q * tid - i) << shift);
        sh_rank[buf] = r - before;
      }
      before += c[i];
    }
    __syncthreads();
    prefix = sh_prefix[buf];
    r = sh_rank[buf];
    pmask |= dm << shift;
  };
  pass(h0, 20, 4096, 0);
  // h0 is free again (its last reads were before pass 1's final barrier)
  for (int i = tid; i < 1024; i += kSelThreads) h0[i] = 0;
  pass(h1, 10, 1024, 1);
  pass(h0, 0, 1024, 0);
  const uint32_t T = prefix;
  // keep the keys above T and the first r keys equal to it, in candidate
  // order; a kept key's slot is (greater before) + min(equal before, r).
  // Rounds of RUN * kSelThreads candidates, thread t the run of RUN from
  // RUN t (its keys loaded together: a wave's runs share a few cache lines),
  // one block scan of each count per round.
  // One round: thread t the run of len_run candidates from base + len_run t
  // (at most RUN, a compile-time bound; the run's keys in k, rl of them real).
  int* slot_of = hist;  // the round's slots (-1: dropped), candidate order
  int gt_carry = 0, eq_carry = 0;
  auto round = [&](auto run_c, int len_run, int base, int rl, const uint32_t* k) {
    constexpr int RUN = decltype(run_c)::value;
    // the ids of the round's write-out, requested before the scan
    const int len = min(len_run * kSelThreads, n - base);
    int ids[RUN];
#pragma unroll
    for (int u = 0; u < RUN; ++u) ids[u] = id_of(c0 + base + min(tid + u * kSelThreads, len - 1));
    int gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < RUN; ++j) {
      gt += (j < rl && k[j] > T) ? 1 : 0;
      eq += (j < rl && k[j] == T) ? 1 : 0;
    }
    // one scan of both counts, packed (a round's totals stay below 2^16);
    // its barriers also order this round's slot stores after the previous
    // round's reads
    int tot;
    const int ex = block_excl_scan<kSelThreads>((gt << 16) | eq, lds, &tot);
    int gt_before = gt_carry + (ex >> 16);
    int eq_before = eq_carry + (ex & 0xffff);
    gt_carry += tot >> 16;
    eq_carry += tot & 0xffff;
#pragma unroll
    for (int j = 0; j < RUN; ++j) {
      if (j < rl) {
        const bool g = k[j] > T, q = k[j] == T;
        slot_of[len_run * tid + j] =
            (g || (q && eq_before < r)) ? o + gt_before + min(eq_before, r) : -1;
        gt_before += g ? 1 : 0;
        eq_before += q ? 1 : 0;
      }
    }
    __syncthreads();
    // write out with consecutive lanes on consecutive candidates (a wave's
    // stores then cover few cache lines)
#pragma unroll
    for (int u = 0; u < RUN; ++u) {
      const int i = tid + u * kSelThreads;
      if (i < len) {
        const int slot = slot_of[i];
        pos[ids[u]] = slot;
        if (slot >= 0) kept[slot] = ids[u];
      }
    }
  };
  if (in_regs) {
    round(std::integral_constant<int, kSelRegKeys>{}, K, 0, cnt, kr);
  } else {
    constexpr int RUN = kSelRunKeys;
    // the next round's keys are requested before this round's scan
    uint32_t k[RUN], kn[RUN];
#pragma unroll
    for (int j = 0; j < RUN; ++j) kn[j] = keys[c0 + min(RUN * tid + j, n - 1)];
    for (int base = 0; base < n; base += RUN * kSelThreads) {
      const int rs = base + RUN * tid;
      const int rl = max(0, min(RUN, n - rs));
#pragma unroll
      for (int j = 0; j < RUN; ++j) {
        k[j] = kn[j];
        kn[j] = keys[c0 + min(rs + RUN * kSelThreads + j, n - 1)];
      }
      round(std::integral_constant<int, RUN>{}, RUN, base, rl, k);
    }
  }
}

__global__ __launch_bounds__(kSelThreads) void k_select(const int32_t* __restrict__ cand_off,
                                                        const int32_t* __restrict__ offsets,
                                                        const uint32_t* __restrict__ keys,
                                                        const int32_t* __restrict__ cand,
                                                        int32_t* __restrict__ pos,
                                                        int32_t* __restrict__ kept, int limit) {
  const int e = blockIdx.x;
  const int c0 = min(cand_off[e], limit);
  const int n = min(cand_off[e + 1], limit) - c0;
  const int o = min(offsets[e], limit);
  const int m = min(offsets[e + 1], limit) - o;
  select_expert(c0, n, o, m, keys, cand, pos, kept);
}

// Selection of a small call in one launch, in place of the bucketing kernels
// and k_select.  One workgroup per expert reads every pair's expert and token
// (N <= kSmallSelN; E * N <= kSmallSelWork bounds the redundant reads, served
// by L2), so each builds the whole expert histogram and the candidate and
// kept offsets itself, with no wait on another workgroup.  It then writes its
// own candidates in pair order with their keys and selects as k_select does.
// Workgroup 0 also writes the offsets, the error word, the row-tile prefix,
// the token offsets and pos = -1 for pairs with an index out of range.
// Thread t reads pairs r * kSelThreads + t (rounds r, coalesced); a round's
// candidates of the expert are ranked by one ballot per wave, and one block
// scan over the ballots' counts, in (round, wave) order, gives each its slot.
// Outputs are those of the bucketing path bit for bit.
// Measured per call (Zipf routings): 18.7 against 25.7 us at 512 pairs, 23.0
// against 29.2 at 8192 pairs over 128 experts, even at 16384, slower at 32768
// (47 against 40: every workgroup reads every pair), hence the bound.
constexpr int kSmallSelN = 8192;
constexpr int64_t kSmallSelWork = 1 << 21;
constexpr int kSmallSelE = 1024;
constexpr int kSmallRounds = kSmallSelN / kSelThreads;  // <= 64: one bit each
static_assert(kSmallRounds <= 64, "one bit per round in a 64-bit mask");

bool select_one_launch_ok(int N, int E) {
  const char* env = getenv("LRM_SELECT_ONE_LAUNCH");
  if (env && env[0] == '0') return false;
  return N <= kSmallSelN && E <= kSmallSelE && (int64_t)E * N <= kSmallSelWork;
}

struct SmallSelArgs {
  int N, T, E;
  const int32_t* token;
  const int32_t* expert;
  const int32_t* quota;  // device [E], or nullptr: qp when use_qp
  const float* score;
  int32_t* cand_off;
  int32_t* offsets;
  int32_t* cand;
  uint32_t* keys;
  int32_t* pos;
  int32_t* kept;
  uint32_t* err;
  int32_t* tok_off;  // or nullptr
  int32_t* mt_off;   // or nullptr
  int mt_bm;
  int64_t max_kept;
  int limit;
  int use_qp;
  QuotaPack qp;
};

__global__ __launch_bounds__(kSelThreads) void k_select_small(SmallSelArgs a) {
  constexpr int NW = kSelThreads / kWave;
  __shared__ int cnt[kSmallSelE];     // candidates per expert
  __shared__ int mcount[kSmallSelE];  // kept per expert (capped by the scan)
  __shared__ int coff[kSmallSelE + 1], koff[kSmallSelE + 1];
  __shared__ uint64_t bal[kSmallRounds * NW];
  __shared__ int bal_off[kSmallRounds * NW + 1];
  __shared__ int lds[NW + 1];
  __shared__ uint32_t eor;
  const int e = blockIdx.x, tid = threadIdx.x, w = tid >> 6, l = lane_id();
  const int N = a.N, T = a.T, E = a.E;
  for (int i = tid; i < E; i += kSelThreads) cnt[i] = 0;
  if (tid == 0) eor = 0u;
  __syncthreads();
  const int R = (N + kSelThreads - 1) / kSelThreads;
  const uint64_t lt = (l == 0) ? 0ull : (~0ull >> (64 - l));  // lanes below this one
  uint64_t mine = 0;  // bit r: pair r * kSelThreads + tid is a candidate of e
  uint32_t bad = 0;
  // rounds in batches of kSmallBatch, every load of a batch issued before
  // the first is used (a round's loads alone would wait one L2 latency each);
  // the token order is checked by workgroup 0 only, the one that writes the
  // error word
  constexpr int kSmallBatch = 8;
  for (int r0 = 0; r0 < R; r0 += kSmallBatch) {
    int exv[kSmallBatch], tkv[kSmallBatch], tpv[kSmallBatch];
#pragma unroll
    for (int u = 0; u < kSmallBatch; ++u) {
      const int p = (r0 + u) * kSelThreads + tid;
      const bool in = r0 + u < R && p < N;
      exv[u] = in ? a.expert[p] : -1;
      tkv[u] = in ? a.token[p] : 0;
      tpv[u] = (e == 0 && in && p > 0) ? a.token[p - 1] : 0;
    }
#pragma unroll
    for (int u = 0; u < kSmallBatch; ++u) {
      const int r = r0 + u;
      if (r >= R) break;  // uniform
      const int p = r * kSelThreads + tid;
      const bool in = p < N;
      const int ex = exv[u], tk = tkv[u];
      bool valid = false;
      if (in) {
        if (ex < 0 || ex >= E) bad |= kErrExpertRange;
        if (tk < 0 || tk >= T) bad |= kErrTokenRange;
        if (e == 0 && p > 0 && tpv[u] > tk) bad |= kErrTokenOrder;
        valid = ex >= 0 && ex < E && tk >= 0 && tk < T;
        if (valid) atomicAdd(&cnt[ex], 1);
        if (e == 0) {
          if (!valid) a.pos[p] = -1;
          if (a.tok_off) token_offsets_at(p, N, T, a.token, a.tok_off);
        }
      }
      const bool hit = valid && ex == e;
      const uint64_t b = __ballot(hit);
      if (l == 0) bal[r * NW + w] = b;
      mine |= (uint64_t)(hit ? 1 : 0) << r;
    }
  }
  if (e == 0 && tid == 0 && a.tok_off) token_offsets_at(N, N, T, a.token, a.tok_off);
  if (bad) atomicOr(&eor, bad);
  __syncthreads();
  // quotas: device array, or by value, or keep all
  for (int i = tid; i < E; i += kSelThreads) {
    const int q = a.quota ? max(a.quota[i], 0) : (a.use_qp ? max(a.qp.q[i], 0) : 0x7fffffff);
    mcount[i] = min(q, cnt[i]);
  }
  block_scan_array<kSelThreads>(E, [&](int i) { return cnt[i]; }, coff, lds);
  __syncthreads();
  const bool over = scan_kept_capped(E, mcount, koff, a.max_kept, lds);
  if (e == 0 && a.mt_off) {
    block_scan_array<kSelThreads>(
        E, [&](int i) { return (mcount[i] + a.mt_bm - 1) / a.mt_bm; }, a.mt_off, lds);
  }
  // slots of the expert's candidates: ballot counts in (round, wave) order
  block_scan_array<kSelThreads>(R * NW, [&](int i) { return __popcll(bal[i]); }, bal_off, lds);
  __syncthreads();
  const int limit = a.limit;
  const int c0 = min(coff[e], limit);
  const int n = min(coff[e + 1], limit) - c0;
  const int o = min(koff[e], limit);
  const int m = min(koff[e + 1], limit) - o;
  for (uint64_t mm = mine; mm; mm &= mm - 1) {
    const int r = __builtin_ctzll(mm);
    const int p = r * kSelThreads + tid;
    const int idx = bal_off[r * NW + w] + __popcll(bal[r * NW + w] & lt);
    if (idx < n) {
      a.cand[c0 + idx] = p;
      a.keys[c0 + idx] = __float_as_uint(a.score[p]);
    }
  }
  if (e == 0) {
    for (int i = tid; i <= E; i += kSelThreads) {
      a.cand_off[i] = coff[i];
      a.offsets[i] = koff[i];
    }
    if (tid == 0) a.err[0] = eor | (over ? kErrCapacity : 0u);
  }
  // the candidates written above are read back by other threads of the block
  __syncthreads();
  select_expert(c0, n, o, m, a.keys, a.cand, a.pos, a.kept);
}

// tok_off[t] = first pair index whose token is >= t, for t in [0, T].
__global__ __launch_bounds__(256) void k_token_offsets(int N, int T,
                                                       const int32_t* __restrict__ token,
                                                       int32_t* __restrict__ tok_off) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p > N) return;
  token_offsets_at(p, N, T, token, tok_off);
}

// mt_off[e] = sum over e' < e of ceil(M_e' / bm)  (row tiles of the dX GEMM)
__global__ __launch_bounds__(kSelThreads) void k_tile_plan(int E, int bm,
                                                           const int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ mt_off) {
  __shared__ int lds[kSelThreads / kWave + 1];
  block_scan_array<kSelThreads>(
      E, [&](int e) { return (offsets[e + 1] - offsets[e] + bm - 1) / bm; }, mt_off, lds);
}

__global__ __launch_bounds__(256) void k_fill_u32(uint32_t* __restrict__ p, uint32_t v,
                                                  int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

// ------------------------------------------------------------- launchers

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  LRM_LAUNCH((unsigned)((n + 255) / 256), 256, 0, s, k_fill_u32)(p, v, n);
  return hipGetLastError();
}

hipError_t launch_bucket_count(int N, int T, int E, const int32_t* token, const int32_t* expert,
                               int32_t* blkcnt, uint32_t* blkerr, int32_t* tok_off,
                               hipStream_t s) {
  if (N <= 0) return hipSuccess;
  const int nblk = bucket_blocks(N);
  if (nblk > kScanTile) return hipErrorInvalidValue;
  LRM_LAUNCH(nblk, 256, E * sizeof(int), s, k_bucket_count)(N, T, E, bucket_chunk(N), token,
                                                            expert, blkcnt, blkerr, tok_off);
  return hipGetLastError();
}

hipError_t launch_bucket(const BucketArgs& a, hipStream_t s) {
  const int nblk = bucket_blocks(a.N);
  const int chunk = bucket_chunk(a.N);
  if (nblk > kScanTile) return hipErrorInvalidValue;
  if (a.N > 0) {
    LRM_LAUNCH(nblk, 256, a.E * sizeof(int), s, k_bucket_count)(a.N, a.T, a.E, chunk, a.token,
                                                        a.expert, a.blkcnt, a.blkerr, a.tok_off);
  }
  if (a.mt_off && a.mt_bm < 1) return hipErrorInvalidValue;
  const bool use_qp = !a.quota && a.qpack;
  if (use_qp && a.E > kQuotaPackMax) return hipErrorInvalidValue;
  const bool rows = a.N > 0 && nblk <= kRowsMaxBlk && (int64_t)a.E * nblk >= kRowsMinWork;
  if (rows) {
    constexpr int per = kSelThreads / kWave;
    LRM_LAUNCH((a.E + per - 1) / per, kSelThreads, 0, s, k_bucket_rows)(nblk, a.E, a.blkcnt,
                                                                          a.cand_off);
  }
  LRM_LAUNCH(1, kSelThreads, 2 * a.E * sizeof(int), s, k_bucket_scan)(
      nblk, a.E, a.blkcnt, a.quota, a.cand_off, a.offsets, a.blkerr, a.err, a.mt_off, a.mt_bm,
      use_qp ? *a.qpack : QuotaPack{}, use_qp ? 1 : 0, a.max_kept, rows ? 1 : 0);
  if (a.N > 0) {
    LRM_LAUNCH(nblk, 64, a.E * sizeof(int), s, k_bucket_scatter)(a.N, a.T, a.E, chunk, a.token,
                                                         a.expert, a.blkcnt, a.cand_off, a.score,
                                                         a.cand, a.keys, a.pos, a.keep_all);
  }
  return hipGetLastError();
}

hipError_t launch_select(int E, const int32_t* cand_off, const int32_t* offsets,
                         const uint32_t* keys, const int32_t* cand, int32_t* pos, int32_t* kept,
                         int limit, hipStream_t s) {
  LRM_LAUNCH(E, kSelThreads, 0, s, k_select)(cand_off, offsets, keys, cand, pos, kept,
                                             limit < 0 ? 0 : limit);
  return hipGetLastError();
}

hipError_t launch_select_one(const BucketArgs& b, int32_t* kept, int limit, hipStream_t s) {
  if (!select_one_launch_ok(b.N, b.E) || b.keep_all || !b.score || !b.keys) return hipErrorInvalidValue;
  if (b.mt_off && b.mt_bm < 1) return hipErrorInvalidValue;
  const bool use_qp = !b.quota && b.qpack;
  if (use_qp && b.E > kQuotaPackMax) return hipErrorInvalidValue;
  SmallSelArgs a{};
  a.N = b.N; a.T = b.T; a.E = b.E; a.token = b.token; a.expert = b.expert;
  a.quota = b.quota; a.score = b.score;
  a.cand_off = b.cand_off; a.offsets = b.offsets; a.cand = b.cand; a.keys = b.keys;
  a.pos = b.pos; a.kept = kept; a.err = b.err; a.tok_off = b.tok_off;
  a.mt_off = b.mt_off; a.mt_bm = b.mt_bm; a.max_kept = b.max_kept;
  a.limit = limit < 0 ? 0 : limit;
  a.use_qp = use_qp ? 1 : 0;
  if (use_qp) a.qp = *b.qpack;
  LRM_LAUNCH(b.E, kSelThreads, 0, s, k_select_small)(a);
  return hipGetLastError();
}

hipError_t launch_kept_offsets(int E, const int32_t* cand_off, const int32_t* quota,
                               const QuotaPack* qpack, int32_t* offsets, uint32_t* err,
                               int64_t cap, hipStream_t s) {
  const bool use_qp = !quota && qpack;
  if (use_qp && E > kQuotaPackMax) return hipErrorInvalidValue;
  if (cap >= 0 && !err) return hipErrorInvalidValue;
  LRM_LAUNCH(1, kSelThreads, E * sizeof(int), s, k_kept_offsets)(E, cand_off, quota, offsets,
                                                   use_qp ? *qpack : QuotaPack{}, use_qp ? 1 : 0,
                                                   err, cap);
  return hipGetLastError();
}

hipError_t launch_token_offsets(int N, int T, const int32_t* token, int32_t* tok_off,
                                hipStream_t s) {
  LRM_LAUNCH((N + 1 + 255) / 256, 256, 0, s, k_token_offsets)(N, T, token, tok_off);
  return hipGetLastError();
}

hipError_t launch_tile_plan(int E, int bm, const int32_t* offsets, int32_t* mt_off,
                            hipStream_t s) {
  LRM_LAUNCH(1, kSelThreads, 0, s, k_tile_plan)(E, bm, offsets, mt_off);
  return hipGetLastError();
}

}  // namespace lrm

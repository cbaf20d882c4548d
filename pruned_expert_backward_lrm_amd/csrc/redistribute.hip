// Redistribution of kept pairs onto replicas, and the receiver-major layout
// of the packed rows (LRMoE page 1, section on what LRMoE does, bullet
// "Перераспределение"; page 2, same section, bullet "Redistribution"; the
// packing by receiver and expert: bullet "Физическое уплотнение").
//
// lrm_redistribute (host): each expert's M_e kept pairs are split over the
// GPUs holding a copy of it, minimising the peak per-GPU load
// base[g] + sum_e x[e][g] (pairs), optionally under per-GPU capacities.  It is
// a transportation problem: the optimum is found exactly by a binary search on
// the peak T, each T checked by a maximum flow source -> expert (M_e) ->
// GPU in R_e -> sink (min(cap_g, T - base_g)), which is integral.  The flow
// is Dinic's algorithm on arrays carved from the caller's host workspace.
//
// lrm_quota_waterfill (host): the controller's quotas before the backward
// pass (bullet "Квоты до вычислений"): water-filling caps under one pair
// budget, the most loaded experts trimmed first.
//
// lrm_receiver_layout (device): given the assignment, the destination of
// every expert-major packed row in a receiver-major buffer: receiver g's block
// holds experts e = 0..E-1 in order, x[e][g] rows each; an expert's rows go
// to its replicas in ascending g.  One planning block (per-expert replica
// prefixes, per-receiver expert prefixes, receiver offsets, validation), then
// one thread per row.
#include <algorithm>

#include "common.h"
#include "launch.h"
#include "lrm.h"

namespace lrm {

constexpr int kPlanThreads = 1024;

// Planning block.  rep_off[e][g] = sum_{g' < g} x[e][g'] (G+1 per expert);
// blk_off[g][e] = sum_{e' < e} x[e'][g] (E+1 per receiver); send_off[g] =
// rows of the receivers before g (G+1).  err[0] = kErrAssign if some x < 0 or
// an expert's shares do not add up to offsets[e+1] - offsets[e], else 0.
__global__ __launch_bounds__(kPlanThreads) void k_layout_plan(int E, int G,
                                                              const int32_t* __restrict__ offsets,
                                                              const int32_t* __restrict__ assign,
                                                              int32_t* __restrict__ rep_off,
                                                              int32_t* __restrict__ send_off,
                                                              int32_t* __restrict__ blk_off,
                                                              uint32_t* __restrict__ err) {
  __shared__ int lds[kPlanThreads / kWave + 1];
  __shared__ uint32_t bad;
  if (threadIdx.x == 0) bad = 0u;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPlanThreads) {
    const int32_t* xe = assign + (int64_t)e * G;
    int32_t* re = rep_off + (int64_t)e * (G + 1);
    int64_t run = 0;
    bool ok = true;
    for (int g = 0; g < G; ++g) {
      const int x = xe[g];
      ok = ok && x >= 0;
      re[g] = (int32_t)min<int64_t>(run, INT32_MAX);
      run += max(x, 0);
    }
    re[G] = (int32_t)min<int64_t>(run, INT32_MAX);
    if (!ok || run != (int64_t)offsets[e + 1] - offsets[e]) atomicOr(&bad, kErrAssign);
  }
  for (int g = 0; g < G; ++g)
    block_scan_array<kPlanThreads>(
        E, [&](int e) { return max(assign[(int64_t)e * G + g], 0); }, blk_off + (int64_t)g * (E + 1),
        lds);
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t s = 0;
    for (int g = 0; g < G; ++g) {
      send_off[g] = (int32_t)min<int64_t>(s, INT32_MAX);
      s += blk_off[(int64_t)g * (E + 1) + E];
    }
    send_off[G] = (int32_t)min<int64_t>(s, INT32_MAX);
    err[0] = bad;
  }
}

// dst[m] for every packed row m < min(offsets[E], max_rows).  With a valid
// assignment dst is a permutation of 0..offsets[E]-1; otherwise (err set) its
// values are unspecified but every access stays inside its array.
__global__ __launch_bounds__(256) void k_layout_rows(int E, int G, int max_rows,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ rep_off,
                                                     const int32_t* __restrict__ send_off,
                                                     const int32_t* __restrict__ blk_off,
                                                     int32_t* __restrict__ dst) {
  const int M = min(offsets[E], max_rows);
  for (int m = blockIdx.x * 256 + threadIdx.x; m < M; m += gridDim.x * 256) {
    // expert: largest e with offsets[e] <= m
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (offsets[mid] <= m) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int j = m - offsets[e];
    const int32_t* re = rep_off + (int64_t)e * (G + 1);
    // replica: largest g < G with re[g] <= j
    int glo = 0, ghi = G;
    while (ghi - glo > 1) {
      const int mid = (glo + ghi) >> 1;
      if (re[mid] <= j) glo = mid; else ghi = mid;
    }
    dst[m] = send_off[glo] + blk_off[(int64_t)glo * (E + 1) + e] + (j - re[glo]);
  }
}

}  // namespace lrm

using namespace lrm;

namespace {

constexpr int kMaxE = 4096;
constexpr int kMaxGpus = 1024;
constexpr size_t kAlign = 256;

// Host arrays of the flow network, carved from the caller's host workspace.
struct Net {
  int V = 0, A = 0;
  int *head, *nxt, *to, *level, *iter, *queue, *pair_arc;
  int64_t *cap, *orig;

  void add(int u, int v, int64_t c) {
    to[A] = v; cap[A] = c; orig[A] = c; nxt[A] = head[u]; head[u] = A++;
    to[A] = u; cap[A] = 0; orig[A] = 0; nxt[A] = head[v]; head[v] = A++;
  }
  bool bfs(int s, int t) {
    std::fill(level, level + V, -1);
    int qh = 0, qt = 0;
    level[s] = 0;
    queue[qt++] = s;
    while (qh < qt) {
      const int u = queue[qh++];
      for (int a = head[u]; a >= 0; a = nxt[a])
        if (cap[a] > 0 && level[to[a]] < 0) {
          level[to[a]] = level[u] + 1;
          queue[qt++] = to[a];
        }
    }
    return level[t] >= 0;
  }
  // One augmenting path in the level graph (iterative, explicit stack in
  // queue[]); returns the flow pushed, 0 if none is left.
  int64_t augment(int s, int t) {
    int depth = 0;
    queue[0] = s;
    while (depth >= 0) {
      const int u = queue[depth];
      if (u == t) {
        int64_t f = INT64_MAX;
        for (int d = 0; d < depth; ++d) f = std::min(f, cap[iter[queue[d]]]);
        for (int d = 0; d < depth; ++d) {
          const int a = iter[queue[d]];
          cap[a] -= f;
          cap[a ^ 1] += f;
        }
        return f;
      }
      int& a = iter[u];
      while (a >= 0 && !(cap[a] > 0 && level[to[a]] == level[u] + 1)) a = nxt[a];
      if (a >= 0) {
        queue[++depth] = to[a];
      } else {
        level[u] = -1;  // dead end: leave it out of this phase
        if (--depth >= 0) iter[queue[depth]] = nxt[iter[queue[depth]]];
      }
    }
    return 0;
  }
  int64_t maxflow(int s, int t) {
    int64_t total = 0;
    while (bfs(s, t)) {
      std::copy(head, head + V, iter);
      for (int64_t f; (f = augment(s, t)) > 0;) total += f;
    }
    return total;
  }
};

// Bump carving of the host workspace (base == nullptr: measure only).
struct HostCarve {
  char* base;
  size_t off = 0;
  explicit HostCarve(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(int64_t n) {
    off = (off + 63) / 64 * 64;
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += (size_t)(n > 0 ? n : 0) * sizeof(T);
    return p;
  }
};

void carve_net(HostCarve& c, int E, int G, Net* n) {
  const int V = E + G + 2;
  const int64_t A = 2 * ((int64_t)E + (int64_t)E * G + G);
  n->V = V;
  n->head = c.take<int>(V);
  n->level = c.take<int>(V);
  n->iter = c.take<int>(V);
  n->queue = c.take<int>(V + 1);
  n->nxt = c.take<int>(A);
  n->to = c.take<int>(A);
  n->pair_arc = c.take<int>((int64_t)E * G);
  n->cap = c.take<int64_t>(A);
  n->orig = c.take<int64_t>(A);
}

// Flow network for peak T; returns whether every kept pair fits.
bool feasible(Net& n, int E, int G, const int32_t* kept, const uint8_t* replica,
              const int64_t* base, const int64_t* cap, int64_t T, int64_t total) {
  const int s = E + G, t = E + G + 1;
  n.A = 0;
  std::fill(n.head, n.head + n.V, -1);
  for (int e = 0; e < E; ++e) n.add(s, e, kept[e]);
  for (int e = 0; e < E; ++e)
    for (int g = 0; g < G; ++g) {
      n.pair_arc[(int64_t)e * G + g] = -1;
      if (replica[(int64_t)e * G + g]) {
        n.pair_arc[(int64_t)e * G + g] = n.A;
        n.add(e, E + g, total);
      }
    }
  for (int g = 0; g < G; ++g) {
    int64_t room = std::max<int64_t>(0, T - (base ? base[g] : 0));
    if (cap) room = std::min(room, cap[g]);
    n.add(E + g, t, room);
  }
  return n.maxflow(s, t) == total;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

size_t lrm_redistribute_workspace_size(int32_t E, int32_t G) {
  if (E < 1 || E > kMaxE || G < 1 || G > kMaxGpus) return 0;
  HostCarve c(nullptr);
  Net n;
  carve_net(c, E, G, &n);
  return (c.off + 63) / 64 * 64;
}

lrm_status lrm_redistribute(int32_t E, int32_t G, const int32_t* kept, const uint8_t* replica,
                            const int64_t* base, const int64_t* cap, int32_t* assign,
                            int64_t* peak, void* host_ws, size_t host_ws_bytes) {
  if (E < 1 || E > kMaxE || G < 1 || G > kMaxGpus) return LRM_ERR_SHAPE;
  if (!kept || !replica || !assign || !peak) return LRM_ERR_NULL;
  if (!host_ws || host_ws_bytes < lrm_redistribute_workspace_size(E, G)) return LRM_ERR_WORKSPACE;
  int64_t total = 0, lo = 0;
  for (int e = 0; e < E; ++e) {
    if (kept[e] < 0) return LRM_ERR_QUOTA;
    total += kept[e];
    bool any = false;
    for (int g = 0; g < G; ++g) any = any || replica[(int64_t)e * G + g] != 0;
    if (kept[e] > 0 && !any) return LRM_ERR_INFEASIBLE;
  }
  for (int g = 0; g < G; ++g) {
    if ((base && base[g] < 0) || (cap && cap[g] < 0)) return LRM_ERR_SHAPE;
    lo = std::max<int64_t>(lo, base ? base[g] : 0);
  }
  HostCarve c(host_ws);
  Net n;
  carve_net(c, E, G, &n);
  int64_t hi = lo + total;
  if (!feasible(n, E, G, kept, replica, base, cap, hi, total)) return LRM_ERR_INFEASIBLE;
  while (lo < hi) {  // smallest feasible peak
    const int64_t mid = lo + (hi - lo) / 2;
    if (feasible(n, E, G, kept, replica, base, cap, mid, total))
      hi = mid;
    else
      lo = mid + 1;
  }
  feasible(n, E, G, kept, replica, base, cap, lo, total);
  for (int e = 0; e < E; ++e)
    for (int g = 0; g < G; ++g) {
      const int a = n.pair_arc[(int64_t)e * G + g];
      assign[(int64_t)e * G + g] = a < 0 ? 0 : (int32_t)(n.orig[a] - n.cap[a]);
    }
  *peak = lo;
  return LRM_OK;
}

lrm_status lrm_quota_waterfill(int32_t E, const int32_t* counts, int64_t budget, int32_t* quota) {
  if (E < 1 || E > kMaxE) return LRM_ERR_SHAPE;
  if (!counts || !quota) return LRM_ERR_NULL;
  if (budget < 0) return LRM_ERR_QUOTA;
  int64_t total = 0;
  int32_t nmax = 0;
  for (int e = 0; e < E; ++e) {
    if (counts[e] < 0) return LRM_ERR_QUOTA;
    total += counts[e];
    nmax = std::max(nmax, counts[e]);
  }
  if (budget >= total) {
    for (int e = 0; e < E; ++e) quota[e] = counts[e];
    return LRM_OK;
  }
  auto kept_at = [&](int64_t tau) {
    int64_t s = 0;
    for (int e = 0; e < E; ++e) s += std::min<int64_t>(counts[e], tau);
    return s;
  };
  int64_t lo = 0, hi = nmax;  // largest tau with kept_at(tau) <= budget
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (kept_at(mid) <= budget) lo = mid; else hi = mid - 1;
  }
  int64_t left = budget - kept_at(lo);
  for (int e = 0; e < E; ++e) {  // (counts may alias quota: read before write)
    const int32_t n = counts[e];
    int32_t q = (int32_t)std::min<int64_t>(n, lo);
    if (left > 0 && n > lo) {
      ++q;
      --left;
    }
    quota[e] = q;
  }
  return LRM_OK;
}

size_t lrm_receiver_layout_workspace_size(int32_t E, int32_t G) {
  if (E < 1 || E > kMaxE || G < 1 || G > kMaxGpus) return 0;
  const size_t err = kAlign;
  const size_t rep = ((size_t)E * (G + 1) * sizeof(int32_t) + kAlign - 1) / kAlign * kAlign;
  return err + rep;
}

lrm_status lrm_receiver_layout(int32_t E, int32_t G, const int32_t* offsets,
                               const int32_t* assign, int32_t max_rows, int32_t* send_off,
                               int32_t* blk_off, int32_t* dst, void* ws, size_t ws_bytes,
                               void* stream) {
  if (E < 1 || E > kMaxE || G < 1 || G > kMaxGpus || max_rows < 0) return LRM_ERR_SHAPE;
  if (!offsets || !assign || !send_off || !blk_off || (max_rows > 0 && !dst)) return LRM_ERR_NULL;
  if (!ws || ws_bytes < lrm_receiver_layout_workspace_size(E, G)) return LRM_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  uint32_t* err = static_cast<uint32_t*>(ws);
  int32_t* rep_off = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + kAlign);
  LRM_LAUNCH(1, kPlanThreads, 0, s, k_layout_plan)(E, G, offsets, assign, rep_off, send_off,
                                                   blk_off, err);
  if (hipGetLastError() != hipSuccess) return LRM_ERR_HIP;
  if (max_rows > 0) {
    const int blocks = std::min(4096, (max_rows + 255) / 256);
    LRM_LAUNCH(blocks, 256, 0, s, k_layout_rows)(E, G, max_rows, offsets, rep_off, send_off,
                                                 blk_off, dst);
    if (hipGetLastError() != hipSuccess) return LRM_ERR_HIP;
  }
  return LRM_OK;
}

}  // extern "C"

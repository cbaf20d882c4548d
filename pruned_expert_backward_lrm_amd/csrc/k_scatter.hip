// Return to the original layout: per-pair input-gradient rows computed on the
// packed blocks are sent back to token (or pair) order, each multiplied by the
// pair's routing weight (LRMoE page 1, bullet "Физическое уплотнение").
//   TOKEN: dX[t] = sum over the kept pairs p of t, in pair order, of
//          w_p * (src_0 row of p + src_1 row of p);  0 if none is kept
//   PAIR:  dX[p] = w_p * (src_0 row of p + src_1 row of p), 0 if dropped
// Deterministic: a fixed summation order, no atomics.  HBM-bound: one wave
// per output row, 16-byte loads and stores.
#include "common.h"
#include "launch.h"

namespace lrm {

// Row of pair p in source k, or -1.  Rows past what the packed buffers hold
// (possible only when a captured call is replayed with other host quotas,
// which the selection flags as an error) are taken as missing.
__device__ __forceinline__ int src_row(const ScatterArgs& a, int k, int p) {
  if (!a.src[k]) return -1;
  int r = a.pos[k][p];
  if (r >= 0 && a.pos2[k]) r = r < a.pos2_rows[k] ? a.pos2[k][r] : -1;
  return r < a.src_rows[k] ? r : -1;
}

__device__ __forceinline__ f32x4 ld4(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}

// Token layout: one wave per (token, block of kUnpCols columns), so that every
// wave has a short dependency chain (offsets -> descriptors -> rows) and the
// whole grid is resident at once.  The token's pair descriptors (source rows,
// weight) are loaded once, one pair per lane, and broadcast with shuffles; the
// rows of kUnpBatch pairs are then loaded together with buffer loads (a pair
// with nothing kept takes an offset outside the bound and reads zeros, so no
// branch stands between the loads) before they are summed in pair order.
constexpr int kUnpChunks = 2;  // 16-byte chunks per lane
constexpr int kUnpCols = kUnpChunks * kWave * 4;
constexpr int kUnpBatch = 4;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const float* p, int64_t nbytes) {
  const int n = nbytes <= 0 ? 0 : (nbytes > 0x7ffffff0ll ? 0x7ffffff0 : (int)nbytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), (short)0, n, 0x00020000);
}

__global__ __launch_bounds__(256) void k_unpermute_token(ScatterArgs a) {
  const int nblk = (a.d + kUnpCols - 1) / kUnpCols;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gw >= (int64_t)a.T * nblk) return;
  const int t = (int)(gw / nblk), cb = (int)(gw % nblk) * kUnpCols;
  const int l = lane_id();
  const int p0 = min(max(a.tok_off[t], 0), a.N);
  const int p1 = min(max(a.tok_off[t + 1], p0), a.N);
  // columns of this lane
  int col[kUnpChunks];
#pragma unroll
  for (int u = 0; u < kUnpChunks; ++u) col[u] = cb + (u * kWave + l) * 4;
  f32x4 acc[kUnpChunks];
#pragma unroll
  for (int u = 0; u < kUnpChunks; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool two = a.src[1] != nullptr;  // a second source (wave-uniform)
  for (int pb = p0; pb < p1; pb += kWave) {
    const int pi = pb + l;
    int r0 = -1, r1 = -1;
    float w = 0.f;
    if (pi < p1) {
      w = a.weight[pi];
      r0 = src_row(a, 0, pi);
      r1 = src_row(a, 1, pi);
    }
    // only the kept pairs, in pair order (a dropped pair adds exact zeros)
    uint64_t kept = __ballot(r0 >= 0 || r1 >= 0);
    while (kept) {
      f32x4 v[kUnpBatch][2][kUnpChunks];
      float wj[kUnpBatch];
#pragma unroll
      for (int jj = 0; jj < kUnpBatch; ++jj) {
        const bool in = kept != 0;
        const int j = in ? __builtin_ctzll(kept) : 0;
        kept &= kept - 1;  // (a no-op once empty)
        wj[jj] = in ? __shfl(w, j, kWave) : 0.f;
        // one buffer resource per source row (wave-uniform): the row itself,
        // or an empty one (loads return zeros) for a missing row
        const int rj[2] = {__builtin_amdgcn_readfirstlane(in ? __shfl(r0, j, kWave) : -1),
                           __builtin_amdgcn_readfirstlane(in ? __shfl(r1, j, kWave) : -1)};
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          if (k == 1 && !two) {
#pragma unroll
            for (int u = 0; u < kUnpChunks; ++u) v[jj][k][u] = f32x4{0.f, 0.f, 0.f, 0.f};
            continue;
          }
          const __amdgpu_buffer_rsrc_t rs =
              rows_rsrc(a.src[k] + (int64_t)max(rj[k], 0) * a.d, rj[k] >= 0 ? (int64_t)a.d * 4 : 0);
#pragma unroll
          for (int u = 0; u < kUnpChunks; ++u)
            v[jj][k][u] = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                           rs, col[u] < a.d ? col[u] * 4 : 0x7ffffff0, 0, 0));
        }
      }
#pragma unroll
      for (int jj = 0; jj < kUnpBatch; ++jj)
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
          for (int u = 0; u < kUnpChunks; ++u) acc[u] += wj[jj] * v[jj][k][u];
    }
  }
  float* out = a.dX + (int64_t)t * a.d;
#pragma unroll
  for (int u = 0; u < kUnpChunks; ++u)
    if (col[u] < a.d) *reinterpret_cast<f32x4*>(out + col[u]) = acc[u];
}

__global__ __launch_bounds__(256) void k_unpermute_pair(ScatterArgs a) {
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (p >= a.N) return;
  const float w = a.weight[p];
  const int r0 = src_row(a, 0, p);
  const int r1 = src_row(a, 1, p);
  float* out = a.dX + (int64_t)p * a.d;
  for (int c = lane_id() * 4; c < a.d; c += kWave * 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (r0 >= 0) acc += w * ld4(a.src[0] + (int64_t)r0 * a.d + c);
    if (r1 >= 0) acc += w * ld4(a.src[1] + (int64_t)r1 * a.d + c);
    *reinterpret_cast<f32x4*>(out + c) = acc;
  }
}

hipError_t launch_unpermute(const ScatterArgs& a, hipStream_t s) {
  if (!a.dX || (!a.out_pair && a.T > 0 && !a.tok_off)) return hipErrorInvalidValue;
  if (a.out_pair) {
    if (a.N > 0) LRM_LAUNCH((a.N + 3) / 4, 256, 0, s, k_unpermute_pair)(a);
  } else {
    const int64_t waves = (int64_t)a.T * ((a.d + kUnpCols - 1) / kUnpCols);
    if (waves > (1ll << 33)) return hipErrorInvalidValue;
    if (a.T > 0) LRM_LAUNCH((unsigned)((waves + 3) / 4), 256, 0, s, k_unpermute_token)(a);
  }
  return hipGetLastError();
}

}  // namespace lrm

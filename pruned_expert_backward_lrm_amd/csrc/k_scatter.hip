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

__device__ __forceinline__ int src_row(const ScatterArgs& a, int k, int p) {
  if (!a.src[k]) return -1;
  int r = a.pos[k][p];
  if (r >= 0 && a.pos2[k]) r = a.pos2[k][r];
  return r;
}

__device__ __forceinline__ f32x4 ld4(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}

// Columns held in registers per pass: kUnpChunks x 64 lanes x 4 floats.
constexpr int kUnpChunks = 8;

// One wave per token.  The token's pair descriptors (source rows, weight) are
// loaded once, one pair per lane, and broadcast with shuffles; each pair then
// issues kUnpChunks independent 16-byte loads per lane.
__global__ __launch_bounds__(256) void k_unpermute_token(ScatterArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int l = lane_id();
  const int p0 = min(max(a.tok_off[t], 0), a.N);
  const int p1 = min(max(a.tok_off[t + 1], p0), a.N);
  float* out = a.dX + (int64_t)t * a.d;
  for (int cb = 0; cb < a.d; cb += kUnpChunks * kWave * 4) {
    f32x4 acc[kUnpChunks];
#pragma unroll
    for (int u = 0; u < kUnpChunks; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int pb = p0; pb < p1; pb += kWave) {
      const int pi = pb + l;
      int r0 = -1, r1 = -1;
      float w = 0.f;
      if (pi < p1) {
        w = a.weight[pi];
        r0 = src_row(a, 0, pi);
        r1 = src_row(a, 1, pi);
      }
      const int np = min(kWave, p1 - pb);
      for (int j = 0; j < np; ++j) {
        const float wj = __shfl(w, j, kWave);
        const int rj0 = __shfl(r0, j, kWave);
        const int rj1 = __shfl(r1, j, kWave);
        if (rj0 >= 0) {
          const float* src = a.src[0] + (int64_t)rj0 * a.d + cb + l * 4;
#pragma unroll
          for (int u = 0; u < kUnpChunks; ++u)
            if (cb + (u * kWave + l) * 4 < a.d) acc[u] += wj * ld4(src + u * kWave * 4);
        }
        if (rj1 >= 0) {
          const float* src = a.src[1] + (int64_t)rj1 * a.d + cb + l * 4;
#pragma unroll
          for (int u = 0; u < kUnpChunks; ++u)
            if (cb + (u * kWave + l) * 4 < a.d) acc[u] += wj * ld4(src + u * kWave * 4);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnpChunks; ++u) {
      const int c = cb + (u * kWave + l) * 4;
      if (c < a.d) *reinterpret_cast<f32x4*>(out + c) = acc[u];
    }
  }
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
    if (a.T > 0) LRM_LAUNCH((a.T + 3) / 4, 256, 0, s, k_unpermute_token)(a);
  }
  return hipGetLastError();
}

}  // namespace lrm

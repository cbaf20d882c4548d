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

__global__ __launch_bounds__(256) void k_unpermute_token(ScatterArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int p0 = min(max(a.tok_off[t], 0), a.N);
  const int p1 = min(max(a.tok_off[t + 1], p0), a.N);
  float* out = a.dX + (int64_t)t * a.d;
  for (int c = lane_id() * 4; c < a.d; c += kWave * 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int p = p0; p < p1; ++p) {
      const float w = a.weight[p];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int r = src_row(a, k, p);
        if (r >= 0) acc += w * ld4(a.src[k] + (int64_t)r * a.d + c);
      }
    }
    *reinterpret_cast<f32x4*>(out + c) = acc;
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

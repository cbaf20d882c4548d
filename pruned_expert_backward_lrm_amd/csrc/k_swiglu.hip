// SwiGLU expert backward between the down and the gate/up projections, with
// the gate and up LRM scores.
//
// For a pair kept by the down stage, u = W_down^T g is the (unscaled)
// gradient of h = silu(a) * b, so the unscaled gradients at the gate and up
// pre-activations are ga = u * b * silu'(a) and gb = u * silu(a), with
// silu'(a) = s (1 + a (1 - s)), s = sigmoid(a).  Each projection is scored on
// its own (the metric is a per-projection estimate: LRMoE page 1, section
// "Что показали эксперименты и где подвох"; metric: bullet "Отбор по метрике
// LRM"):  s_gate = w^2 |ga|^2 |x|^2,  s_up = w^2 |gb|^2 |x|^2.
//
// One wave per down-kept row; u is read in fp32, a and b in the input dtype;
// ga and gb are written in the input dtype for the next grouped GEMM; the norms
// accumulate the unrounded fp32 values in fp64.  HBM-bound.
#include "common.h"
#include "launch.h"

namespace lrm {

__device__ __forceinline__ void glu_elem(float u, float a, float b, float& ga, float& gb) {
  const float s = sigmoidf_acc(a);
  ga = u * b * (s * (1.0f + a * (1.0f - s)));
  gb = u * (a * s);
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_glu_bwd(GluBwdArgs g) {
  const int M = min(g.offsets_down[g.E], g.max_rows);
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  const int p = g.kept_down[m];
  const int t = g.token[p];
  const float* urow = g.U + (int64_t)m * g.I;
  double sg = 0.0, su = 0.0;
  if constexpr (BF16) {
    const u32x4* ar = reinterpret_cast<const u32x4*>((const uint16_t*)g.A + (int64_t)p * g.lda);
    const u32x4* br = reinterpret_cast<const u32x4*>((const uint16_t*)g.B + (int64_t)p * g.ldb);
    const int64_t ldg = g.ldg > 0 ? g.ldg : g.I;
    u32x4* gar = reinterpret_cast<u32x4*>((uint16_t*)g.GA + (int64_t)m * ldg);
    u32x4* gbr = reinterpret_cast<u32x4*>((uint16_t*)g.GB + (int64_t)m * ldg);
    for (int c = lane_id(); c < g.I / 8; c += kWave) {
      const u32x4 va = ar[c], vb = br[c];
      const f32x4 u0 = *reinterpret_cast<const f32x4*>(urow + c * 8);
      const f32x4 u1 = *reinterpret_cast<const f32x4*>(urow + c * 8 + 4);
      const float uu[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
      u32x4 oa, ob;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float ga0, gb0, ga1, gb1;
        glu_elem(uu[2 * i], bf16_lo(va[i]), bf16_lo(vb[i]), ga0, gb0);
        glu_elem(uu[2 * i + 1], bf16_hi(va[i]), bf16_hi(vb[i]), ga1, gb1);
        sg = fma((double)ga0, (double)ga0, sg);
        sg = fma((double)ga1, (double)ga1, sg);
        su = fma((double)gb0, (double)gb0, su);
        su = fma((double)gb1, (double)gb1, su);
        oa[i] = pack_bf16x2(ga0, ga1);
        ob[i] = pack_bf16x2(gb0, gb1);
      }
      gar[c] = oa;
      gbr[c] = ob;
    }
  } else {
    const float* ar = (const float*)g.A + (int64_t)p * g.lda;
    const float* br = (const float*)g.B + (int64_t)p * g.ldb;
    const int64_t ldg = g.ldg > 0 ? g.ldg : g.I;
    float* gar = (float*)g.GA + (int64_t)m * ldg;
    float* gbr = (float*)g.GB + (int64_t)m * ldg;
    for (int c = lane_id() * 4; c < g.I; c += kWave * 4) {
      const f32x4 va = *reinterpret_cast<const f32x4*>(ar + c);
      const f32x4 vb = *reinterpret_cast<const f32x4*>(br + c);
      const f32x4 vu = *reinterpret_cast<const f32x4*>(urow + c);
      f32x4 oa, ob;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float ga, gb;
        glu_elem(vu[i], va[i], vb[i], ga, gb);
        sg = fma((double)ga, (double)ga, sg);
        su = fma((double)gb, (double)gb, su);
        oa[i] = ga;
        ob[i] = gb;
      }
      *reinterpret_cast<f32x4*>(gar + c) = oa;
      *reinterpret_cast<f32x4*>(gbr + c) = ob;
    }
  }
  sg = wave_sum(sg);
  su = wave_sum(su);
  if (lane_id() == 0 && (g.s_gate || g.s_up)) {
    const double w = g.weight[p];
    const double x2 = g.x_pair ? g.x2[p] : g.x2[t];
    if (g.s_gate) g.s_gate[m] = (float)(w * w * sg * x2);
    if (g.s_up) g.s_up[m] = (float)(w * w * su * x2);
  }
}

hipError_t launch_glu_bwd(const GluBwdArgs& g, hipStream_t s) {
  if (g.max_rows <= 0) return hipSuccess;
  if (!g.offsets_down || !g.kept_down || !g.U || !g.A || !g.B || !g.GA || !g.GB ||
      ((g.s_gate || g.s_up) && !g.x2) || (g.ldg != 0 && g.ldg < g.I))
    return hipErrorInvalidValue;
  const int blocks = (g.max_rows + 3) / 4;
  if (g.bf16)
    LRM_LAUNCH(blocks, 256, 0, s, k_glu_bwd<true>)(g);
  else
    LRM_LAUNCH(blocks, 256, 0, s, k_glu_bwd<false>)(g);
  return hipGetLastError();
}

}  // namespace lrm

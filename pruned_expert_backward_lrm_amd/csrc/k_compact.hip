// Physical compaction: kept gradient and activation rows are gathered into
// dense per-expert blocks, expert after expert, with no padding (LRMoE page 1,
// section on what LRMoE does, bullet "Физическое уплотнение"), or, through a
// row map, into dense blocks per receiver and expert (the same bullet).  The routing
// weight is folded into the activation side here (Xp = w x), so the grouped
// GEMM computes dW_e = Gp_e^T Xp_e directly.
//
// HBM-bound row copy: one wave per packed row, 16-byte loads and stores, a
// row's loads issued before its stores.
#include "common.h"
#include "launch.h"

namespace lrm {

__device__ __forceinline__ u32x4 scale_chunk_bf16(u32x4 v, float w) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(bf16_lo(v[i]) * w, bf16_hi(v[i]) * w);
  return o;
}
__device__ __forceinline__ u32x4 scale_chunk_f32(u32x4 v, float w) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(__uint_as_float(v[i]) * w);
  return o;
}

// w * silu(a) * b for one 16-byte chunk of a and b
__device__ __forceinline__ u32x4 glu_chunk_bf16(u32x4 va, u32x4 vb, float w) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a0 = bf16_lo(va[i]), a1 = bf16_hi(va[i]);
    const float h0 = a0 / (1.0f + expf(-a0)) * bf16_lo(vb[i]);
    const float h1 = a1 / (1.0f + expf(-a1)) * bf16_hi(vb[i]);
    o[i] = pack_bf16x2(w * h0, w * h1);
  }
  return o;
}
__device__ __forceinline__ u32x4 glu_chunk_f32(u32x4 va, u32x4 vb, float w) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float av = __uint_as_float(va[i]);
    const float h = av / (1.0f + expf(-av)) * __uint_as_float(vb[i]);
    o[i] = __float_as_uint(w * h);
  }
  return o;
}

// One row of nch 16-byte chunks, f applied per chunk; each lane loads up to
// kCpBatch chunks before it stores any, so a row's loads are in flight
// together.
constexpr int kCpBatch = 8;
template <class F>
__device__ __forceinline__ void copy_row(u32x4* dst, const u32x4* src, int nch, F f) {
  const int l = lane_id();
  for (int c0 = 0; c0 < nch; c0 += kCpBatch * kWave) {
    u32x4 v[kCpBatch];
#pragma unroll
    for (int i = 0; i < kCpBatch; ++i) {
      const int c = c0 + i * kWave + l;
      if (c < nch) v[i] = src[c];
    }
#pragma unroll
    for (int i = 0; i < kCpBatch; ++i) {
      const int c = c0 + i * kWave + l;
      if (c < nch) dst[c] = f(v[i]);
    }
  }
}
template <class F>
__device__ __forceinline__ void copy_row2(u32x4* dst, const u32x4* src, const u32x4* src2,
                                          int nch, F f) {
  const int l = lane_id();
  for (int c0 = 0; c0 < nch; c0 += kCpBatch / 2 * kWave) {
    u32x4 va[kCpBatch / 2], vb[kCpBatch / 2];
#pragma unroll
    for (int i = 0; i < kCpBatch / 2; ++i) {
      const int c = c0 + i * kWave + l;
      if (c < nch) {
        va[i] = src[c];
        vb[i] = src2[c];
      }
    }
#pragma unroll
    for (int i = 0; i < kCpBatch / 2; ++i) {
      const int c = c0 + i * kWave + l;
      if (c < nch) dst[c] = f(va[i], vb[i]);
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_compact(CompactArgs a) {
  constexpr int kEsz = BF16 ? 2 : 4;
  constexpr int kEpc = 16 / kEsz;
  const int M = min(a.offsets[a.E], a.max_rows);
  const int nw = gridDim.x * 4;
  for (int j = blockIdx.x * 4 + (threadIdx.x >> 6); j < M; j += nw) {
    const int o = a.dst ? a.dst[j] : j;  // output row (wave-uniform)
    if (o < 0 || o >= a.max_rows) continue;
    const int id = a.kept[j];
    const int p = a.pairmap ? a.pairmap[id] : id;
    const int t = a.token[p];
    if (a.Xp) {
      const float w = a.weight[p];
      const int64_t xr = (a.x_pair || a.glu) ? (int64_t)p : (int64_t)t;
      const u32x4* src = reinterpret_cast<const u32x4*>((const char*)a.X + xr * a.ldx * kEsz);
      u32x4* dst = reinterpret_cast<u32x4*>((char*)a.Xp + (int64_t)o * a.xcols * kEsz);
      if (a.glu) {
        const u32x4* src2 =
            reinterpret_cast<const u32x4*>((const char*)a.X2 + xr * a.ldx2 * kEsz);
        copy_row2(dst, src, src2, a.xcols / kEpc, [w](u32x4 va, u32x4 vb) {
          return BF16 ? glu_chunk_bf16(va, vb, w) : glu_chunk_f32(va, vb, w);
        });
      } else {
        copy_row(dst, src, a.xcols / kEpc,
                 [w](u32x4 v) { return BF16 ? scale_chunk_bf16(v, w) : scale_chunk_f32(v, w); });
      }
    }
    if (a.Gp) {
      const int64_t gr = a.g_by_id ? (int64_t)id : (a.g_pair ? (int64_t)p : (int64_t)t);
      const u32x4* src = reinterpret_cast<const u32x4*>((const char*)a.G + gr * a.ldg * kEsz);
      u32x4* dst = reinterpret_cast<u32x4*>((char*)a.Gp + (int64_t)o * a.gcols * kEsz);
      copy_row(dst, src, a.gcols / kEpc, [](u32x4 v) { return v; });
    }
  }
}

// One thread per packed row: the source row and routing weight of each kept
// row, for a GEMM loader that gathers and scales the rows itself.
__global__ __launch_bounds__(256) void k_row_map(CompactArgs a, int32_t* __restrict__ xrow,
                                                 float* __restrict__ xw) {
  const int M = min(a.offsets[a.E], a.max_rows);
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= M) return;
  const int id = a.kept[j];
  const int p = a.pairmap ? a.pairmap[id] : id;
  xrow[j] = a.x_pair ? p : a.token[p];
  xw[j] = a.weight[p];
}

hipError_t launch_row_map(const CompactArgs& a, int32_t* xrow, float* xw, hipStream_t s) {
  if (a.max_rows <= 0) return hipSuccess;
  if (!a.offsets || !a.kept || !a.token || !a.weight || !xrow || !xw) return hipErrorInvalidValue;
  LRM_LAUNCH((a.max_rows + 255) / 256, 256, 0, s, k_row_map)(a, xrow, xw);
  return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  if (a.max_rows <= 0 || (!a.Xp && !a.Gp)) return hipSuccess;
  if (!a.offsets || !a.kept || !a.token || !a.weight) return hipErrorInvalidValue;
  if ((a.Xp && !a.X) || (a.Gp && !a.G) || (a.glu && !a.X2)) return hipErrorInvalidValue;
  const int64_t want = ((int64_t)a.max_rows + 3) / 4;
  const int blocks = (int)(want < (1 << 16) ? want : (1 << 16));
  if (a.bf16)
    LRM_LAUNCH(blocks, 256, 0, s, k_compact<true>)(a);
  else
    LRM_LAUNCH(blocks, 256, 0, s, k_compact<false>)(a);
  return hipGetLastError();
}

}  // namespace lrm

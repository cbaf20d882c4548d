// LRM score kernels.
//
// The score of a pair is the squared Frobenius norm of its weight-gradient
// contribution (w g) x^T, which factorises as w^2 |g|^2 |x|^2 (LRMoE page 1,
// section on what LRMoE does, bullet "Отбор по метрике LRM").  Each factor is
// a row sum of squares: TOKEN-layout rows are reduced once per token into an
// fp64 table; PAIR-layout rows are reduced inline by one wave per pair.  All
// sums are fp64; the product is formed in fp64 and rounded once to fp32.
//
// HBM-bound: every input element is read exactly once (16-byte loads, one
// wave per row, 64-lane fp64 tree reduction).
#include "common.h"
#include "launch.h"

namespace lrm {

// Sum of squares of a 16-byte chunk, accumulated in fp64.
__device__ __forceinline__ double chunk_sumsq_bf16(u32x4 v, double acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    double lo = bf16_lo(v[i]), hi = bf16_hi(v[i]);
    acc = fma(lo, lo, acc);
    acc = fma(hi, hi, acc);
  }
  return acc;
}
__device__ __forceinline__ double chunk_sumsq_f32(u32x4 v, double acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    double f = __uint_as_float(v[i]);
    acc = fma(f, f, acc);
  }
  return acc;
}

template <bool BF16>
__device__ __forceinline__ double row_sumsq_wave(const char* row, int cols) {
  constexpr int kEpc = BF16 ? 8 : 4;  // elements per 16-byte chunk
  const int nchunks = cols / kEpc;
  const u32x4* r = reinterpret_cast<const u32x4*>(row);
  double acc = 0.0;
  for (int c = lane_id(); c < nchunks; c += kWave) {
    u32x4 v = __builtin_nontemporal_load(r + c);
    acc = BF16 ? chunk_sumsq_bf16(v, acc) : chunk_sumsq_f32(v, acc);
  }
  return wave_sum(acc);
}

// out[r] = sum_j M[r][j]^2 (fp64), one wave per row.
template <bool BF16>
__global__ __launch_bounds__(256) void k_row_sumsq(const char* __restrict__ M, int64_t ld_bytes,
                                                   int cols, int rows, double* __restrict__ out) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  double s = row_sumsq_wave<BF16>(M + (int64_t)r * ld_bytes, cols);
  if (lane_id() == 0) out[r] = s;
}

// h = silu(a) * b for one 16-byte chunk of a and b; returns sum of h^2.
__device__ __forceinline__ double glu_chunk_sumsq_bf16(u32x4 a, u32x4 b, double acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a0 = bf16_lo(a[i]), a1 = bf16_hi(a[i]);
    float h0 = a0 / (1.0f + expf(-a0)) * bf16_lo(b[i]);
    float h1 = a1 / (1.0f + expf(-a1)) * bf16_hi(b[i]);
    acc = fma((double)h0, (double)h0, acc);
    acc = fma((double)h1, (double)h1, acc);
  }
  return acc;
}
__device__ __forceinline__ double glu_chunk_sumsq_f32(u32x4 a, u32x4 b, double acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float av = __uint_as_float(a[i]);
    float h = av / (1.0f + expf(-av)) * __uint_as_float(b[i]);
    acc = fma((double)h, (double)h, acc);
  }
  return acc;
}

// Per-pair score with inline reductions of PAIR-layout operands.
//   g factor: gtab[token[p]] (table) or |G row p|^2 (inline)
//   x factor: xtab[row]      (table) or |X row p|^2 (inline)
//             or |silu(A row p) * B row p|^2       (GLU inline)
struct PairScoreArgs {
  int N, T;
  const int32_t* token;
  const float* weight;
  const char* G; int64_t ldg_bytes; int gcols; const double* gtab; int g_pair;
  const char* X; int64_t ldx_bytes; int xcols; const double* xtab; int x_pair;
  const char* A; const char* B; int64_t lda_bytes, ldb_bytes; int icols;
  float* score;
};

// XMODE: 0 = table, 1 = inline row, 2 = inline GLU.  GINL: g inline.
template <bool BF16, bool GINL, int XMODE>
__global__ __launch_bounds__(256) void k_pair_score_wave(PairScoreArgs a) {
  const int64_t p = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (p >= a.N) return;
  const int t = a.token[p];
  const bool tok_ok = (t >= 0 && t < a.T);
  double g2, x2;
  if constexpr (GINL) {
    g2 = row_sumsq_wave<BF16>(a.G + p * a.ldg_bytes, a.gcols);
  } else {
    g2 = a.g_pair ? a.gtab[p] : (tok_ok ? a.gtab[t] : 0.0);
  }
  if constexpr (XMODE == 1) {
    x2 = row_sumsq_wave<BF16>(a.X + p * a.ldx_bytes, a.xcols);
  } else if constexpr (XMODE == 2) {
    constexpr int kEpc = BF16 ? 8 : 4;
    const u32x4* ra = reinterpret_cast<const u32x4*>(a.A + p * a.lda_bytes);
    const u32x4* rb = reinterpret_cast<const u32x4*>(a.B + p * a.ldb_bytes);
    double acc = 0.0;
    for (int c = lane_id(); c < a.icols / kEpc; c += kWave) {
      u32x4 va = __builtin_nontemporal_load(ra + c);
      u32x4 vb = __builtin_nontemporal_load(rb + c);
      acc = BF16 ? glu_chunk_sumsq_bf16(va, vb, acc) : glu_chunk_sumsq_f32(va, vb, acc);
    }
    x2 = wave_sum(acc);
  } else {
    x2 = a.x_pair ? a.xtab[p] : (tok_ok ? a.xtab[t] : 0.0);
  }
  if (lane_id() == 0) {
    const double w = a.weight[p];
    a.score[p] = (float)(w * w * g2 * x2);  // an out-of-range token gave a zero factor
  }
}

// Per-pair score when both factors come from tables: one thread per pair.
__global__ __launch_bounds__(256) void k_pair_score_table(PairScoreArgs a) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= a.N) return;
  const int t = a.token[p];
  const bool tok_ok = (t >= 0 && t < a.T);
  if (!tok_ok) { a.score[p] = 0.0f; return; }
  const double g2 = a.g_pair ? a.gtab[p] : a.gtab[t];
  const double x2 = a.x_pair ? a.xtab[p] : a.xtab[t];
  const double w = a.weight[p];
  a.score[p] = (float)(w * w * g2 * x2);
}

hipError_t launch_row_sumsq(const void* M, int bf16, int64_t ld, int cols, int rows,
                            double* out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int esz = bf16 ? 2 : 4;
  dim3 grid((rows + 3) / 4);
  if (bf16)
    LRM_LAUNCH(grid, 256, 0, s, k_row_sumsq<true>)((const char*)M, ld * esz, cols, rows, out);
  else
    LRM_LAUNCH(grid, 256, 0, s, k_row_sumsq<false>)((const char*)M, ld * esz, cols, rows, out);
  return hipGetLastError();
}

template <bool BF16>
static void dispatch_pair_score(const PairScoreArgs& a, int g_inline, int x_mode, hipStream_t s) {
  dim3 wgrid((a.N + 3) / 4);
  if (!g_inline && x_mode == 0) {
    LRM_LAUNCH((a.N + 255) / 256, 256, 0, s, k_pair_score_table)(a);
  } else if (g_inline && x_mode == 0) {
    LRM_LAUNCH(wgrid, 256, 0, s, k_pair_score_wave<BF16, true, 0>)(a);
  } else if (g_inline && x_mode == 1) {
    LRM_LAUNCH(wgrid, 256, 0, s, k_pair_score_wave<BF16, true, 1>)(a);
  } else if (!g_inline && x_mode == 1) {
    LRM_LAUNCH(wgrid, 256, 0, s, k_pair_score_wave<BF16, false, 1>)(a);
  } else if (g_inline && x_mode == 2) {
    LRM_LAUNCH(wgrid, 256, 0, s, k_pair_score_wave<BF16, true, 2>)(a);
  } else {
    LRM_LAUNCH(wgrid, 256, 0, s, k_pair_score_wave<BF16, false, 2>)(a);
  }
}

hipError_t launch_pair_score(const ScoreOperands& op, hipStream_t s) {
  if (op.N <= 0) return hipSuccess;
  const int esz = op.bf16 ? 2 : 4;
  PairScoreArgs a{};
  a.N = op.N; a.T = op.T; a.token = op.token; a.weight = op.weight;
  a.G = (const char*)op.G; a.ldg_bytes = op.ldg * esz; a.gcols = op.gcols; a.gtab = op.gtab;
  a.g_pair = op.g_pair;
  a.X = (const char*)op.X; a.ldx_bytes = op.ldx * esz; a.xcols = op.xcols; a.xtab = op.xtab;
  a.x_pair = op.x_pair;
  a.A = (const char*)op.A; a.B = (const char*)op.B; a.lda_bytes = op.lda * esz;
  a.ldb_bytes = op.ldb * esz; a.icols = op.icols;
  a.score = op.score;
  // a PAIR operand without a precomputed table is reduced inline
  const int g_inline = op.g_pair && op.gtab == nullptr;
  const int x_mode = op.glu ? 2 : ((op.x_pair && op.xtab == nullptr) ? 1 : 0);
  if (op.bf16)
    dispatch_pair_score<true>(a, g_inline, x_mode, s);
  else
    dispatch_pair_score<false>(a, g_inline, x_mode, s);
  return hipGetLastError();
}

}  // namespace lrm

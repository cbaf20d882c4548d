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

// silu(a) = a / (1 + e^-a) in fp32, within a few ulp, in about half the
// instructions of expf and an IEEE divide (the GLU score pass is bound by
// this arithmetic, not by its loads):
//   e^-a = 2^t 2^c with t = -a log2(e) rounded to fp32 and c its rounding
//   error (an fma, plus the low part of log2(e)), 2^c ~ 1 + c ln 2 (|c| <
//   2^-17); 2^t by the hardware exp2 (v_exp_f32);
//   1 / (1 + e^-a) by the hardware reciprocal and one Newton step, e^-a
//   capped at 2^126 so that its reciprocal stays a normal number (below
//   a = -87, where the cap applies, |silu(a)| < 2^-120: a negligible term of
//   a sum of squares).
__device__ __forceinline__ float silu_f32(float a) {
  const float kL = 1.44269502f, kLlo = 1.92596299e-8f, kLn2 = 0.693147181f;
  const float t = -a * kL;
  const float c = fmaf(-a, kL, -t) - a * kLlo;
  const float e = fminf(__builtin_amdgcn_exp2f(t) * fmaf(c, kLn2, 1.0f), 8.50705917e37f);
  const float d = 1.0f + e;
  float r = __builtin_amdgcn_rcpf(d);
  r = fmaf(r, fmaf(-d, r, 1.0f), r);
  return a * r;
}

// h = silu(a) * b for one 16-byte chunk of a and b; returns sum of h^2.
__device__ __forceinline__ double glu_chunk_sumsq_bf16(u32x4 a, u32x4 b, double acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float h0 = silu_f32(bf16_lo(a[i])) * bf16_lo(b[i]);
    float h1 = silu_f32(bf16_hi(a[i])) * bf16_hi(b[i]);
    acc = fma((double)h0, (double)h0, acc);
    acc = fma((double)h1, (double)h1, acc);
  }
  return acc;
}
__device__ __forceinline__ double glu_chunk_sumsq_f32(u32x4 a, u32x4 b, double acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float h = silu_f32(__uint_as_float(a[i])) * __uint_as_float(b[i]);
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

// A wave scores kPairsPerWave consecutive pairs.  Rows of up to 128 16-byte
// chunks (1024 bf16 or 512 fp32 columns) are loaded two chunks per lane for
// all of the wave's pairs before any is reduced, and the pairs' token,
// weight and table entries are requested alongside, so a wave waits for
// memory about once rather than once per pair.  Longer rows fall back to a
// chunk loop per pair.
constexpr int kPairsPerWave = 4;

template <bool BF16>
__device__ __forceinline__ double chunk_sumsq(u32x4 v, double acc) {
  return BF16 ? chunk_sumsq_bf16(v, acc) : chunk_sumsq_f32(v, acc);
}

// |row|^2 partial sums of kPairsPerWave rows (lane-local; reduce afterwards).
template <bool BF16>
__device__ __forceinline__ void rows_sumsq_lane(const char* base, int64_t ld_bytes, int cols,
                                                int64_t p0, int npairs, double (&acc)[kPairsPerWave]) {
  constexpr int kEpc = BF16 ? 8 : 4;
  const int nchunks = cols / kEpc;
  const int l = lane_id();
  if (nchunks <= 2 * kWave) {
    u32x4 v[kPairsPerWave][2];
#pragma unroll
    for (int u = 0; u < kPairsPerWave; ++u) {
      const u32x4* r = reinterpret_cast<const u32x4*>(base + (p0 + u) * ld_bytes);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = l + h * kWave;
        v[u][h] = (u < npairs && c < nchunks) ? __builtin_nontemporal_load(r + c)
                                              : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < kPairsPerWave; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[u] = chunk_sumsq<BF16>(v[u][h], acc[u]);
  } else {
#pragma unroll
    for (int u = 0; u < kPairsPerWave; ++u) {
      if (u >= npairs) break;
      const u32x4* r = reinterpret_cast<const u32x4*>(base + (p0 + u) * ld_bytes);
      for (int c = l; c < nchunks; c += kWave)
        acc[u] = chunk_sumsq<BF16>(__builtin_nontemporal_load(r + c), acc[u]);
    }
  }
}

// XMODE: 0 = table, 1 = inline row, 2 = inline GLU.  GINL: g inline.
template <bool BF16, bool GINL, int XMODE>
__global__ __launch_bounds__(256) void k_pair_score_wave(PairScoreArgs a) {
  const int64_t p0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kPairsPerWave;
  if (p0 >= a.N) return;
  const int np = (int)min<int64_t>(kPairsPerWave, a.N - p0);
  const int l = lane_id();
  // lane u < np: pair p0 + u's token, weight and table factors
  int t = -1;
  double w = 0.0, gt = 0.0, xt = 0.0;
  if (l < np) {
    const int64_t p = p0 + l;
    t = a.token[p];
    w = a.weight[p];
    const bool tok_ok = t >= 0 && t < a.T;
    if constexpr (!GINL) gt = a.g_pair ? a.gtab[p] : (tok_ok ? a.gtab[t] : 0.0);
    if constexpr (XMODE == 0) xt = a.x_pair ? a.xtab[p] : (tok_ok ? a.xtab[t] : 0.0);
  }
  double g2[kPairsPerWave], x2[kPairsPerWave];
#pragma unroll
  for (int u = 0; u < kPairsPerWave; ++u) g2[u] = x2[u] = 0.0;
  if constexpr (GINL) rows_sumsq_lane<BF16>(a.G, a.ldg_bytes, a.gcols, p0, np, g2);
  if constexpr (XMODE == 1) rows_sumsq_lane<BF16>(a.X, a.ldx_bytes, a.xcols, p0, np, x2);
  if constexpr (XMODE == 2) {
    // A and B rows pair by pair (batching them across pairs costs occupancy)
    constexpr int kEpc = BF16 ? 8 : 4;
#pragma unroll
    for (int u = 0; u < kPairsPerWave; ++u) {
      if (u >= np) break;
      const u32x4* ra = reinterpret_cast<const u32x4*>(a.A + (p0 + u) * a.lda_bytes);
      const u32x4* rb = reinterpret_cast<const u32x4*>(a.B + (p0 + u) * a.ldb_bytes);
      for (int c = l; c < a.icols / kEpc; c += kWave) {
        u32x4 va = __builtin_nontemporal_load(ra + c);
        u32x4 vb = __builtin_nontemporal_load(rb + c);
        x2[u] = BF16 ? glu_chunk_sumsq_bf16(va, vb, x2[u]) : glu_chunk_sumsq_f32(va, vb, x2[u]);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kPairsPerWave; ++u) {
    if (u >= np) break;
    const double gu = GINL ? wave_sum(g2[u]) : __shfl(gt, u, kWave);
    const double xu = XMODE != 0 ? wave_sum(x2[u]) : __shfl(xt, u, kWave);
    const double wu = __shfl(w, u, kWave);
    const int tu = __shfl(t, u, kWave);
    // an out-of-range token gives a zero factor, as in the table path
    const bool tok_ok = tu >= 0 && tu < a.T;
    if (l == 0) a.score[p0 + u] = (float)(wu * wu * gu * (tok_ok || XMODE != 0 ? xu : 0.0));
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
  dim3 wgrid((unsigned)((a.N + 4 * kPairsPerWave - 1) / (4 * kPairsPerWave)));
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

// Variable-size grouped GEMM on the packed per-expert blocks, no zero padding
// (LRMoE page 1, section on what LRMoE does, bullet "Физическое уплотнение").
// For each expert e with M_e packed rows (device-side sizes, no host sync):
//   dW[e] = Gp_e^T Xp_e   [d_out][d_in], K = M_e (zero tile when M_e = 0)
//   dXp_e = Gp_e W_e (+ Gp2_e W2_e)  [M_e][d_in], K = d_out (+ d_out2)
// Both products run in one launch over a combined tile list: E * (d_out/BM) *
// (d_in/BN) fixed-size dW tiles, then dX tiles (ceil(M_e/BM) row tiles per
// expert, located by a binary search of a device-built prefix).  Block ids are
// remapped so that consecutive tiles (the same expert) land on the same XCD
// and share its L2.
//
// bf16: v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  128x128 tile, BK 64,
// 4 waves as 2x2, each wave 64x64 = 4x4 MFMA blocks.  Operands are staged in
// LDS as [row][k] (k contiguous, XOR-swizzled 128-byte rows) so that each
// lane's fragment (8 consecutive k) is one 16-byte LDS read.  Sources whose k
// runs along rows (Gp and Xp in dW, W in dX) are loaded as 4x8 blocks with
// 16-byte global loads and transposed in registers before the LDS store.  Two
// LDS stages; global loads run two k-tiles ahead of the MFMAs.
// The MFMA is issued with the N-side fragment first, so each lane's four
// accumulators are four consecutive output columns (one 16-byte store).
//
// fp32: plain LDS-tiled fp32 FMA (64x64 tile) for fp32 inputs.
#include "common.h"
#include "launch.h"

namespace lrm {

constexpr int BM = 128, BN = 128, BK = 64, NT = 256;

__device__ __forceinline__ int xcd_remap(int b, int G) {
  // hardware places block b on XCD b % 8; give each XCD a contiguous range
  return (b & 7) * (G >> 3) + (b >> 3);
}

// Largest e with mt_off[e] <= mt (mt < mt_off[E]).
__device__ __forceinline__ int find_expert(const int32_t* mt_off, int E, int mt) {
  int lo = 0, hi = E;  // invariant: mt_off[lo] <= mt < mt_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (mt_off[mid] <= mt) lo = mid; else hi = mid;
  }
  return lo;
}

// The two tile kinds are interleaved along the logical order so that every
// XCD receives its proportional share of both: position L holds dX tile c(L)
// when c(L+1) > c(L), with c(L) = floor(L * nX / (nW + nX)), and dW tile
// L - c(L) otherwise (a bijection onto both tile lists).
__device__ __forceinline__ bool is_dx_tile(int L, int nW, int nX, int* idx) {
  const int64_t T = (int64_t)nW + nX;
  const int c0 = (int)(((int64_t)L * nX) / T);
  const int c1 = (int)(((int64_t)(L + 1) * nX) / T);
  if (c1 > c0) {
    *idx = c0;
    return true;
  }
  *idx = L - c0;
  return false;
}

// ------------------------------------------------------------------ bf16

// LDS operand tile: 128 rows x 64 k (bf16), 128-byte rows, no padding.  The
// 8-byte half-granules of row r are XOR-swizzled by 2*((r & 7) ^ ((r>>3) & 7))
// (an even value, so 16-byte granules stay contiguous): the 16-byte fragment
// reads (16 consecutive rows) and the transposed 8-byte stores (rows 8 apart)
// both spread over all banks.
__device__ __forceinline__ int lds_off(int r, int h) {
  return r * BK + ((h ^ (((r & 7) ^ ((r >> 3) & 7)) << 1)) << 2);
}

struct Regs { u32x4 v[4]; };

// k-contiguous source: tile rows r in [0,128) at src + r*ld, k in [k0,k0+64)
__device__ __forceinline__ void load_direct(Regs& R, const uint16_t* src, int64_t ld,
                                            int rows_valid, int k0, int K) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = threadIdx.x + q * NT;
    const int r = idx >> 3, k = k0 + (idx & 7) * 8;
    R.v[q] = (r < rows_valid && k < K)
                 ? *reinterpret_cast<const u32x4*>(src + (int64_t)r * ld + k)
                 : u32x4{0u, 0u, 0u, 0u};
  }
}
__device__ __forceinline__ void store_direct(const Regs& R, uint16_t* lds) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = threadIdx.x + q * NT;
    const int r = idx >> 3, kc = idx & 7;
    *reinterpret_cast<u32x4*>(lds + lds_off(r, 2 * kc)) = R.v[q];
  }
}

// k-strided source: element (k, n) at src + k*ld + n.  Thread owns k rows
// kg*4..kg*4+3 and columns ng*8..ng*8+7 of the 64x128 tile.
__device__ __forceinline__ void load_trans(Regs& R, const uint16_t* src, int64_t ld, int k0,
                                           int kend, int n0, int ncols) {
  const int kg = threadIdx.x >> 4, ng = threadIdx.x & 15;
  const int n = n0 + ng * 8;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int k = k0 + kg * 4 + r;
    R.v[r] = (k < kend && n < ncols)
                 ? *reinterpret_cast<const u32x4*>(src + (int64_t)k * ld + n)
                 : u32x4{0u, 0u, 0u, 0u};
  }
}
__device__ __forceinline__ uint32_t pick_half(uint32_t x, uint32_t y, int hi) {
  return hi ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
}
__device__ __forceinline__ void store_trans(const Regs& R, uint16_t* lds) {
  const int kg = threadIdx.x >> 4, ng = threadIdx.x & 15;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int w = c >> 1, h = c & 1;
    u32x2 o;
    o[0] = pick_half(R.v[0][w], R.v[1][w], h);
    o[1] = pick_half(R.v[2][w], R.v[3][w], h);
    *reinterpret_cast<u32x2*>(lds + lds_off(ng * 8 + c, kg)) = o;
  }
}

struct TileSrc {
  // A side (output rows): direct (dX: Gp rows) or transposed (dW: Gp columns)
  const uint16_t* a; int64_t lda; int a_rows_valid; int a_n0; int a_ncols;
  // B side (output columns): always transposed
  const uint16_t* b; int64_t ldb; int b_n0; int b_ncols;
  int K;  // k extent of this segment (rows valid for the transposed sources)
};

template <bool A_DIRECT>
__device__ __forceinline__ void load_tile(Regs& RA, Regs& RB, const TileSrc& s, int k0) {
  if constexpr (A_DIRECT)
    load_direct(RA, s.a, s.lda, s.a_rows_valid, k0, s.K);
  else
    load_trans(RA, s.a, s.lda, k0, s.K, s.a_n0, s.a_ncols);
  load_trans(RB, s.b, s.ldb, k0, s.K, s.b_n0, s.b_ncols);
}
template <bool A_DIRECT>
__device__ __forceinline__ void store_tile(const Regs& RA, const Regs& RB, uint16_t* As,
                                           uint16_t* Bs) {
  if constexpr (A_DIRECT) store_direct(RA, As); else store_trans(RA, As);
  store_trans(RB, Bs);
}

// Field-wise select (keeps both descriptors in registers).
__device__ __forceinline__ TileSrc pick_seg(const TileSrc& x, const TileSrc& y, bool first) {
  TileSrc r;
  r.a = first ? x.a : y.a;
  r.lda = first ? x.lda : y.lda;
  r.a_rows_valid = first ? x.a_rows_valid : y.a_rows_valid;
  r.a_n0 = first ? x.a_n0 : y.a_n0;
  r.a_ncols = first ? x.a_ncols : y.a_ncols;
  r.b = first ? x.b : y.b;
  r.ldb = first ? x.ldb : y.ldb;
  r.b_n0 = first ? x.b_n0 : y.b_n0;
  r.b_ncols = first ? x.b_ncols : y.b_ncols;
  r.K = first ? x.K : y.K;
  return r;
}

// One output tile: the K segments s0 and (if nseg == 2) s1 are summed.
// Two LDS stages: while the MFMAs consume stage kt & 1, the registers holding
// k-tile kt+1 are stored into the other stage and the global loads of k-tile
// kt+2 are issued; one barrier per k-tile.
template <bool A_DIRECT>
__device__ __forceinline__ void mma_tile(const TileSrc& s0, const TileSrc& s1, int nseg, float* C,
                                         int64_t ldc, int rows_valid, int cols_valid,
                                         uint16_t* As, uint16_t* Bs) {
  const int l = lane_id(), w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk0 = (s0.K + BK - 1) / BK;
  const int nk1 = nseg > 1 ? (s1.K + BK - 1) / BK : 0;
  const int total = nk0 + nk1;
  auto k_of = [&](int t) { return (t < nk0 ? t : t - nk0) * BK; };

  Regs RA, RB;
  if (total > 0) {
    load_tile<A_DIRECT>(RA, RB, pick_seg(s0, s1, 0 < nk0), 0);
    store_tile<A_DIRECT>(RA, RB, As, Bs);
    if (total > 1) load_tile<A_DIRECT>(RA, RB, pick_seg(s0, s1, 1 < nk0), k_of(1));
    __syncthreads();
  }
  for (int kt = 0; kt < total; ++kt) {
    const int cur = (kt & 1) * (BM * BK);
    const uint16_t* Ac = As + cur;
    const uint16_t* Bc = Bs + cur;
#pragma unroll
    for (int kk = 0; kk < BK / 8; kk += 4) {
      bf16x8 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 64 + i * 16 + (l & 15);
        af[i] = *reinterpret_cast<const bf16x8*>(Ac + lds_off(row, 2 * (kk + (l >> 4))));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = wn * 64 + j * 16 + (l & 15);
        bf[j] = *reinterpret_cast<const bf16x8*>(Bc + lds_off(col, 2 * (kk + (l >> 4))));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < total) {
      const int nxt = ((kt + 1) & 1) * (BM * BK);
      store_tile<A_DIRECT>(RA, RB, As + nxt, Bs + nxt);
      if (kt + 2 < total)
        load_tile<A_DIRECT>(RA, RB, pick_seg(s0, s1, kt + 2 < nk0), k_of(kt + 2));
    }
    __syncthreads();
  }
  // lane holds C[row = .. + (l & 15)][col = .. + (l >> 4) * 4 + 0..3]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wm * 64 + i * 16 + (l & 15);
    if (row >= rows_valid) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = wn * 64 + j * 16 + (l >> 4) * 4;
      if (col < cols_valid) *reinterpret_cast<f32x4*>(C + (int64_t)row * ldc + col) = acc[i][j];
    }
  }
}

struct GemmPlan {
  GemmArgs a;
  int ntm_w, ntn, nW, nX, G;
};

__global__ __launch_bounds__(NT) void k_grouped_gemm_bf16(GemmPlan P) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2 * BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2 * BN * BK];
  const GemmArgs& a = P.a;
  const int L = xcd_remap(blockIdx.x, P.G);
  if (L >= P.nW + P.nX) return;
  int idx;
  const bool dx = is_dx_tile(L, P.nW, P.nX, &idx);
  if (!dx) {
    const int per = P.ntm_w * P.ntn;
    const int e = idx / per, rem = idx % per;
    const int i0 = (rem / P.ntn) * BM, j0 = (rem % P.ntn) * BN;
    const int kb = a.offsets[e];
    const int Me = max(0, min(a.offsets[e + 1], a.max_rows) - kb);
    TileSrc s;
    s.a = (const uint16_t*)a.Gp + (int64_t)kb * a.d_out; s.lda = a.d_out;
    s.a_rows_valid = 0; s.a_n0 = i0; s.a_ncols = a.d_out;
    s.b = (const uint16_t*)a.Xp + (int64_t)kb * a.d_in; s.ldb = a.d_in;
    s.b_n0 = j0; s.b_ncols = a.d_in;
    s.K = Me;
    float* C = a.dW + (int64_t)e * a.d_out * a.d_in + (int64_t)i0 * a.d_in + j0;
    mma_tile<false>(s, s, 1, C, a.d_in, min(BM, a.d_out - i0), min(BN, a.d_in - j0), As, Bs);
    return;
  }
  const int mt = idx / P.ntn, tn = idx % P.ntn;
  if (mt >= a.mt_off[a.E]) return;
  const int e = find_expert(a.mt_off, a.E, mt);
  const int m0 = a.offsets[e] + (mt - a.mt_off[e]) * BM;
  const int rows = min(BM, min(a.offsets[e + 1], a.max_rows) - m0);
  if (rows <= 0) return;
  const int j0 = tn * BN;
  TileSrc s0, s1;
  s0.a = (const uint16_t*)a.Gp + (int64_t)m0 * a.d_out; s0.lda = a.d_out;
  s0.a_rows_valid = rows; s0.a_n0 = 0; s0.a_ncols = 0;
  s0.b = (const uint16_t*)a.W + (int64_t)e * a.w_stride; s0.ldb = a.d_in;
  s0.b_n0 = j0; s0.b_ncols = a.d_in;
  s0.K = a.d_out;
  s1 = s0;
  int nseg = 1;
  if (a.Gp2) {
    s1.a = (const uint16_t*)a.Gp2 + (int64_t)m0 * a.d_out2; s1.lda = a.d_out2;
    s1.b = (const uint16_t*)a.W2 + (int64_t)e * a.w2_stride;
    s1.K = a.d_out2;
    nseg = 2;
  }
  float* C = a.dXp + (int64_t)m0 * a.d_in + j0;
  mma_tile<true>(s0, s1, nseg, C, a.d_in, rows, min(BN, a.d_in - j0), As, Bs);
}

// ------------------------------------------------------------------ fp32

constexpr int FBM = 64, FBN = 64, FBK = 16;

// A(m, k) and B(k, n) element fetchers for the two tile kinds.
struct F32Seg {
  const float* a; int64_t lda; int a_trans;  // a_trans: A(m,k) = a[k*lda + m]
  const float* b; int64_t ldb;               // B(k,n) = b[k*ldb + n]
  int K; int a_rows_valid; int a_ncols; int b_ncols;
};

__device__ void f32_tile(const F32Seg& s0, const F32Seg& s1, int nseg, float* C, int64_t ldc,
                         int rows_valid, int cols_valid, int m0, int n0) {
  __shared__ float As[FBK][FBM + 1];
  __shared__ float Bs[FBK][FBN + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int s = 0; s < nseg; ++s) {
    const F32Seg& g = s == 0 ? s0 : s1;
    for (int k0 = 0; k0 < g.K; k0 += FBK) {
      for (int i = threadIdx.x; i < FBK * FBM; i += NT) {
        const int kk = i / FBM, mm = i % FBM;
        const int k = k0 + kk;
        float av = 0.f;
        if (k < g.K) {
          if (g.a_trans) {
            if (m0 + mm < g.a_ncols) av = g.a[(int64_t)k * g.lda + m0 + mm];
          } else {
            if (mm < g.a_rows_valid) av = g.a[(int64_t)mm * g.lda + k];
          }
        }
        As[kk][mm] = av;
        const int nn = mm;
        float bv = 0.f;
        if (k < g.K && n0 + nn < g.b_ncols) bv = g.b[(int64_t)k * g.ldb + n0 + nn];
        Bs[kk][nn] = bv;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < FBK; ++kk) {
        float av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx * 4 + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty * 4 + i;
    if (r >= rows_valid) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = tx * 4 + j;
      if (c < cols_valid) C[(int64_t)r * ldc + c] = acc[i][j];
    }
  }
}

__global__ __launch_bounds__(NT) void k_grouped_gemm_f32(GemmPlan P) {
  const GemmArgs& a = P.a;
  const int L = xcd_remap(blockIdx.x, P.G);
  if (L >= P.nW + P.nX) return;
  int idx;
  const bool dx = is_dx_tile(L, P.nW, P.nX, &idx);
  if (!dx) {
    const int per = P.ntm_w * P.ntn;
    const int e = idx / per, rem = idx % per;
    const int i0 = (rem / P.ntn) * FBM, j0 = (rem % P.ntn) * FBN;
    const int kb = a.offsets[e];
    const int Me = max(0, min(a.offsets[e + 1], a.max_rows) - kb);
    F32Seg s;
    s.a = (const float*)a.Gp + (int64_t)kb * a.d_out; s.lda = a.d_out; s.a_trans = 1;
    s.b = (const float*)a.Xp + (int64_t)kb * a.d_in; s.ldb = a.d_in;
    s.K = Me; s.a_rows_valid = 0; s.a_ncols = a.d_out; s.b_ncols = a.d_in;
    float* C = a.dW + (int64_t)e * a.d_out * a.d_in + (int64_t)i0 * a.d_in + j0;
    f32_tile(s, s, 1, C, a.d_in, min(FBM, a.d_out - i0), min(FBN, a.d_in - j0), i0, j0);
    return;
  }
  const int mt = idx / P.ntn, tn = idx % P.ntn;
  if (mt >= a.mt_off[a.E]) return;
  const int e = find_expert(a.mt_off, a.E, mt);
  const int m0 = a.offsets[e] + (mt - a.mt_off[e]) * FBM;
  const int rows = min(FBM, min(a.offsets[e + 1], a.max_rows) - m0);
  if (rows <= 0) return;
  const int j0 = tn * FBN;
  F32Seg s0, s1;
  s0.a = (const float*)a.Gp + (int64_t)m0 * a.d_out; s0.lda = a.d_out; s0.a_trans = 0;
  s0.b = (const float*)a.W + (int64_t)e * a.w_stride; s0.ldb = a.d_in;
  s0.K = a.d_out; s0.a_rows_valid = rows; s0.a_ncols = 0; s0.b_ncols = a.d_in;
  s1 = s0;
  int nseg = 1;
  if (a.Gp2) {
    s1.a = (const float*)a.Gp2 + (int64_t)m0 * a.d_out2; s1.lda = a.d_out2;
    s1.b = (const float*)a.W2 + (int64_t)e * a.w2_stride;
    s1.K = a.d_out2;
    nseg = 2;
  }
  float* C = a.dXp + (int64_t)m0 * a.d_in + j0;
  f32_tile(s0, s1, nseg, C, a.d_in, rows, min(FBN, a.d_in - j0), 0, j0);
}

// ------------------------------------------------------------- launcher

int gemm_row_tile(int bf16) { return bf16 ? BM : FBM; }

hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t s) {
  if (!a.offsets || (a.dXp && (!a.W || !a.mt_off || !a.Gp)) || (a.dW && !a.Gp) ||
      (a.dW && a.max_rows > 0 && !a.Xp) || (a.Gp2 && !a.W2))
    return hipErrorInvalidValue;
  const int tm = a.bf16 ? BM : FBM, tn = a.bf16 ? BN : FBN;
  GemmPlan P{};
  P.a = a;
  P.ntn = (a.d_in + tn - 1) / tn;
  P.ntm_w = (a.d_out + tm - 1) / tm;
  P.nW = a.dW ? a.E * P.ntm_w * P.ntn : 0;
  P.nX = (a.dXp && a.max_rows > 0) ? ((a.max_rows + tm - 1) / tm + a.E) * P.ntn : 0;
  if (P.nX > 0) {
    hipError_t err = launch_tile_plan(a.E, tm, a.offsets, a.mt_off, s);
    if (err != hipSuccess) return err;
  }
  const int64_t total = (int64_t)P.nW + P.nX;
  if (total == 0) return hipSuccess;
  if (total > (1ll << 30)) return hipErrorInvalidValue;
  P.G = (int)((total + 7) & ~7ll);
  if (a.bf16)
    LRM_LAUNCH(P.G, NT, 0, s, k_grouped_gemm_bf16)(P);
  else
    LRM_LAUNCH(P.G, NT, 0, s, k_grouped_gemm_f32)(P);
  return hipGetLastError();
}

}  // namespace lrm

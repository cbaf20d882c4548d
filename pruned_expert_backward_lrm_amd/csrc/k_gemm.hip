// Variable-size grouped GEMM on the packed per-expert blocks, no zero padding
// (LRMoE page 1, section on what LRMoE does, bullet "Физическое уплотнение").
// For each expert e with M_e packed rows (device-side sizes, no host sync):
//   dW[e] = Gp_e^T Xp_e   [d_out][d_in], K = M_e (zero tile when M_e = 0)
//   dXp_e = Gp_e W_e (+ Gp2_e W2_e)  [M_e][d_in], K = d_out (+ d_out2)
//
// bf16: two launches of k_gemm_stream, one over the dW tiles (E x d_out/BM x
// d_in/BN, fixed size) and one over the dX tiles (ceil(M_e/BM) row tiles per
// expert, located by a binary search of a device-built prefix).  Each launch
// cuts its tile list into 8 shares of equal cost, one per XCD (block b runs on
// XCD b mod 8); inside a share, persistent blocks run their tiles' k-tiles as
// one stream (or, for MFMA-bound launches of few rounds, one block per tile).
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation, BK 64, tiles of 256x256,
// 256x128, 128x128 and 64x256.  Operands are staged in LDS as [row][k] (k
// contiguous, 128-byte rows with a bank-aware granule swizzle) so that each
// lane's fragment (8 consecutive k) is one 16-byte LDS read.  Sources whose k
// runs along rows (Gp and Xp in dW, W in dX) are loaded as 4x8 blocks with
// 16-byte buffer loads and transposed in registers (v_perm) before the LDS
// store.  Two LDS stages; global loads run up to two k-tiles ahead of the
// MFMAs.  The MFMA is issued with the N-side fragment first, so each lane's
// four accumulators are four consecutive output columns (one 16-byte store,
// or 8 bytes when dW is stored as bf16).  An opt-in variant of the 256x256
// kernels (LRM_GEMM_DMA) loads operand tiles straight into LDS and reads the
// k-strided ones with gfx950's transposing LDS reads instead.
//
// fp32: plain LDS-tiled fp32 FMA (64x64 tile), one launch over the combined
// dW and dX tile list.
#include <stdlib.h>

#include <algorithm>
#include <atomic>

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace lrm {

constexpr int NT = 256;  // threads of an fp32 block

// Read of the per-expert tables (kept offsets, dX row-tile prefix) that no
// GEMM kernel writes.  Through the constant address space a wave-uniform index
// becomes a scalar load, which waits on its own counter; a vector load would
// also wait for every store the wave issued before it (one counter covers
// vector loads and stores, retired in order), so the first table read after a
// tile's stores would hold the wave until those stores reach the cache.
#ifdef LRM_CPU_EMU
__device__ __forceinline__ int ld_table(const int32_t* p, int i) { return p[i]; }
#else
typedef const __attribute__((address_space(4))) int32_t* table_ptr;
__device__ __forceinline__ int ld_table(const int32_t* p, int i) {
  return ((table_ptr)(uintptr_t)p)[i];
}
#endif

__device__ __forceinline__ int xcd_remap(int b, int G) {
  // hardware places block b on XCD b % 8; give each XCD a contiguous range
  return (b & 7) * (G >> 3) + (b >> 3);
}

// Largest e with mt_off[e] <= mt (mt < mt_off[E]).
__device__ __forceinline__ int find_expert(const int32_t* mt_off, int E, int mt) {
  int lo = 0, hi = E;  // invariant: mt_off[lo] <= mt < mt_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ld_table(mt_off, mid) <= mt) lo = mid; else hi = mid;
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

// Grouped raster over an nr x nc tile grid (the dW tiles of one expert):
// tiles are taken kRasterH rows at a time, column by column, so the tiles
// resident on one XCD at any moment (a window of consecutive positions) share
// a few row panels and a few column panels in its L2 instead of one row panel
// and every column panel.
constexpr int kRasterH = 4;
__device__ __forceinline__ void raster(int t, int nr, int nc, int* r, int* c) {
  const int r0 = t / (kRasterH * nc) * kRasterH;
  const int gh = min(kRasterH, nr - r0);
  const int rem = t - r0 * nc;
  *r = r0 + rem % gh;
  *c = rem / gh;
}

// dX tiles (row tiles of all experts, back to back, x nc column tiles): the
// row tiles of one expert are taken kDxGroup at a time, in groups aligned to
// the expert's first row tile, column by column.  The tiles of a group that
// read one column panel of W_e then run side by side on one XCD and share it
// in its L2; groups of a fixed height over the concatenated rows straddle
// experts, and each straddled expert's panel comes from HBM once per group.
// Returns the expert of the tile (row tile mt, column tile tn).
constexpr int kDxGroup = 8;
__device__ __forceinline__ int dx_raster(const int32_t* mt_off, int E, int t, int nc, int* mt,
                                         int* tn) {
  const int m = t / nc;  // a row tile of the group that holds position t
  const int e = find_expert(mt_off, E, m);
  const int e0 = ld_table(mt_off, e);
  const int g0 = e0 + (m - e0) / kDxGroup * kDxGroup;
  const int gh = min(kDxGroup, ld_table(mt_off, e + 1) - g0);
  const int rem = t - g0 * nc;
  *mt = g0 + rem % gh;
  *tn = rem / gh;
  return e;
}

// ------------------------------------------------------------------ bf16

// A block tile configuration: BM x BN outputs, k-tiles of 64, WGM x WGN waves,
// each wave owning a TM x TN sub-tile of FM x FN 16x16 MFMA blocks.
template <int BM_, int BN_, int WGM_, int WGN_, int MINB_ = 1, int STAGES_ = 2>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64;
  static constexpr int MINB = MINB_;      // resident blocks per CU the registers must allow
  static constexpr int STAGES = STAGES_;  // LDS stages (1: two barriers per k-tile)
  static constexpr int WGM = WGM_, WGN = WGN_, NW = WGM_ * WGN_, NT = 64 * NW;
  static constexpr int WPE = (MINB * NW + 3) / 4;  // waves per SIMD (launch bound)
  static constexpr int TM = BM / WGM, TN = BN / WGN;
  static constexpr int FM = TM / 16, FN = TN / 16;
  // A fragments held at once (fewer when two blocks share a CU's registers)
  static constexpr int FCH = (MINB > 1 && FM > 4) ? 4 : FM;
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile");
};

// LDS operand tile: R rows x 64 k (bf16), 128-byte rows, no padding.  The
// 16-byte granule G of row r sits at granule G ^ f(r), with f built from row
// bits as (r4, r3, r1 ^ r5).  On gfx950 a ds_read_b128 is served in four
// passes of 16 lanes ({0-3, 12-15, 20-23, 24-27}, {4-7, 8-11, 16-19, 28-31}
// and the same +32) over 64 four-byte banks, and a ds_write_b64 in passes of
// 16 consecutive lanes over 32 banks (both measured with bank-conflict
// counters).  With this f the fragment reads (16 consecutive rows, granules
// g and g+1 in a pass) and the transposed 8-byte stores (16 lanes: 8 rows 8
// apart x both halves of a granule) hit 16 distinct bank slots per pass.
constexpr int BK = 64;
__device__ __forceinline__ int lds_swz(int r) {
  return ((r >> 4) & 1) | (r & 8) >> 2 | (((r >> 1) ^ (r >> 5)) & 1) << 2;
}
// element offset of 8-byte half-granule h (0..15) of row r
__device__ __forceinline__ int lds_off(int r, int h) {
  return r * BK + ((h ^ (lds_swz(r) << 1)) << 2);
}

// Operand panels are read with buffer loads: a buffer resource per k-tile
// (scalar base and byte bound) plus per-lane byte offsets fixed for the whole
// output tile.  Loads past the bound return zero in hardware, which pads the
// k tail of a segment and the rows past an expert's block without any
// per-lane masking or address arithmetic inside the k loop.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ rsrc_t make_rsrc(const char* base, int64_t nbytes) {
  const int n = nbytes <= 0 ? 0 : (nbytes > 0x7ffffff0ll ? 0x7ffffff0 : (int)nbytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, n, kRsrcWord3);
}
// AUX: cache policy of the load (0 default, kStreamAux non-temporal)
template <int AUX = 0>
__device__ __forceinline__ u32x4 bload(rsrc_t r, int off) {
  return (u32x4)__builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
}
constexpr int kStreamAux = 2;  // the nt bit

// Row panel, k contiguous (dX: Gp rows of one expert): row r at
// base + r*ld, k-tile [k0, k0+64).  Bytes valid: rows_valid rows.
template <int R, int NT>
struct DirectTile {
  static constexpr int Q = (R * 8 + NT - 1) / NT;
  u32x4 v[Q];
  int off[Q];
  __device__ __forceinline__ void init(int64_t ld) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int idx = threadIdx.x + q * NT;
      off[q] = idx < R * 8 ? (int)(((idx >> 3) * ld + (idx & 7) * 8) * 2) : 0x7ffffff0;
    }
  }
  // k0: first k of the tile; K: k extent of the panel (zero past it: a lane
  // whose 8 columns start at or past K takes an offset outside the bound)
  __device__ __forceinline__ void load(const char* base, int64_t ld, int rows_valid, int k0,
                                       int K) {
    const rsrc_t rs = make_rsrc(base + (int64_t)k0 * 2, (int64_t)rows_valid * ld * 2 - k0 * 2);
    const bool tail = k0 + (int)(threadIdx.x & 7) * 8 >= K;  // NT % 8 == 0
#pragma unroll
    for (int q = 0; q < Q; ++q) v[q] = bload(rs, tail ? 0x7ffffff0 : off[q]);
  }
  __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int idx = threadIdx.x + q * NT;
      if ((R * 8) % NT == 0 || idx < R * 8)  // (threadIdx.x < NT)
        *reinterpret_cast<u32x4*>(lds + lds_off(idx >> 3, 2 * (idx & 7))) = v[q];
    }
  }
};

// Two bf16 from the same half of x and y: (x.lo, y.lo) or (x.hi, y.hi), x in
// the low half of the result.  One v_perm_b32 (bytes of y are 4..7).
__device__ __forceinline__ uint32_t pick_half(uint32_t x, uint32_t y, int hi) {
  return __builtin_amdgcn_perm(y, x, hi ? 0x07060302u : 0x05040100u);
}

// k-strided panel, R columns (dW: Gp and Xp columns; dX: W columns): element
// (k, n) at base + k*ld + n, columns [n0, n0+R), rows k < kend valid.  The
// tile is cut into 4(k) x 8(n) blocks, each read with four 16-byte loads and
// transposed in registers into eight 8-byte LDS stores (rows n, 4 k each).
// AUX: cache policy of the loads.
template <int R, int NT, int AUX = 0>
struct TransTile {
  static constexpr int NB = 16 * (R / 8);  // blocks per tile
  static constexpr int Q = (NB + NT - 1) / NT;
  static constexpr int NHI = R / 64;         // groups of 8 column blocks
  static_assert(R % 64 == 0, "transposed tile width");
  u32x4 v[Q][4];
  int off[Q];
  // Block b -> (k group kg of 4 rows, column group ng of 8).  Lanes 0-7 take 8
  // column groups, lane bit 3 the k-group parity, so each 16-lane store pass
  // covers both halves of a granule (see lds_swz).
  __device__ __forceinline__ static void block_of(int b, int* kg, int* ng) {
    *ng = (b & 7) + 8 * ((b >> 4) % NHI);
    *kg = ((b >> 3) & 1) + 2 * ((b >> 4) / NHI);
  }
  __device__ __forceinline__ void init(int64_t ld) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int b = threadIdx.x + q * NT;
      int kg, ng;
      block_of(b, &kg, &ng);
      off[q] = b < NB ? (int)((kg * 4 * ld + ng * 8) * 2) : 0x7ffffff0;
    }
  }
  // stream: the loads take the AUX policy (otherwise the default one)
  __device__ __forceinline__ void load(const char* base, int64_t ld, int k0, int kend, int n0,
                                       bool stream = false) {
    const rsrc_t rs = make_rsrc(base + ((int64_t)k0 * ld + n0) * 2,
                                (int64_t)(kend - k0) * ld * 2 - (int64_t)n0 * 2);
    const int row = (int)(ld * 2);
    if (AUX != 0 && stream) {
#pragma unroll
      for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[q][r] = bload<AUX>(rs, off[q] + r * row);
    } else {
#pragma unroll
      for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[q][r] = bload<0>(rs, off[q] + r * row);
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int b = threadIdx.x + q * NT;
      if (NB % NT != 0 && b >= NB) continue;  // (threadIdx.x < NT)
      int kg, ng;
      block_of(b, &kg, &ng);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int w = c >> 1, h = c & 1;
        u32x2 o;
        o[0] = pick_half(v[q][0][w], v[q][1][w], h);
        o[1] = pick_half(v[q][2][w], v[q][3][w], h);
        *reinterpret_cast<u32x2*>(lds + lds_off(ng * 8 + c, kg)) = o;
      }
    }
  }
};

// The B panel of dW gathered from its source rows: packed row k of B is
// w_k * src[row_k] rounded to bf16 (what compaction would have stored), so no
// packed copy is written or read.  The same 4(k) x 8(n) blocks and register
// transposition as TransTile; each of a lane's four rows has its own source
// row and weight, read from the row map of the k-tile.  Rows at or past kend
// load zeros.  src rows are addressed with 32-bit byte offsets (the host
// keeps src under 2 GiB).
template <int R, int NT>
struct GatherTile {
  using T = TransTile<R, NT>;
  static constexpr int Q = T::Q;
  u32x4 v[Q][4];
  float w[Q][4];
  int kgq[Q], col[Q];  // k group of the lane's block, byte offset of its 8 columns
  // the row map of the next load, requested one load ahead (prefetch()), so
  // that the X rows of a k-tile do not wait for their row indices
  int nrow[Q][4];
  float nw[Q][4];
  __device__ __forceinline__ void init(int64_t) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int b = threadIdx.x + q * NT;
      int kg, ng;
      T::block_of(b, &kg, &ng);
      kgq[q] = b < T::NB ? kg : 1 << 20;  // (threadIdx.x < NT: every lane has a block)
      col[q] = ng * 8 * 2;
    }
  }
  // the row map of k-tile k0 of a segment, for the next load(); rows at or
  // past kend get -1 (zeros)
  __device__ __forceinline__ void prefetch(const int32_t* rows, const float* wts, int k0,
                                           int kend) {
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int k = k0 + kgq[q] * 4 + r;
        const bool ok = k < kend;
        nrow[q][r] = ok ? rows[k] : -1;
        nw[q][r] = ok ? wts[k] : 0.f;
      }
  }
  // the X rows of the k-tile whose row map the last prefetch() requested
  __device__ __forceinline__ void load(const char* src, int64_t ld, int64_t src_rows, int n0) {
    const rsrc_t rs = make_rsrc(src, src_rows * ld * 2);
    const int rb = (int)(ld * 2);
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        w[q][r] = nw[q][r];
        v[q][r] = bload(rs, nrow[q][r] >= 0 ? nrow[q][r] * rb + n0 * 2 + col[q] : 0x7ffffff0);
      }
  }
  __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int b = threadIdx.x + q * NT;
      if (T::NB % NT != 0 && b >= T::NB) continue;
      int kg, ng;
      T::block_of(b, &kg, &ng);
      u32x4 s[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s[r][i] = pack_bf16x2(bf16_lo(v[q][r][i]) * w[q][r], bf16_hi(v[q][r][i]) * w[q][r]);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int wd = c >> 1, h = c & 1;
        u32x2 o;
        o[0] = pick_half(s[0][wd], s[1][wd], h);
        o[1] = pick_half(s[2][wd], s[3][wd], h);
        *reinterpret_cast<u32x2*>(lds + lds_off(ng * 8 + c, kg)) = o;
      }
    }
  }
};

// One K segment of an output tile.  A panel: direct (dX: Gp rows, k
// contiguous) or transposed (dW: Gp columns); B panel: always transposed.
// Both segments of a dual-K tile share the leading dimensions.
struct TileSrc {
  const char* a; const char* b;
  int a_rows_valid;  // direct A: rows of the tile inside the expert's block
  int a_n0, b_n0;    // transposed panels: first column of the tile
  int K;             // k extent (direct: columns of A; transposed: valid rows)
  const int32_t* brow; const float* bw;  // gathered B: row map of the expert's rows
  int stream;  // dX: the expert has one row tile, its W panel is read once
};

__device__ __forceinline__ TileSrc pick_seg(const TileSrc& x, const TileSrc& y, bool first) {
  TileSrc r;
  r.a = first ? x.a : y.a;
  r.b = first ? x.b : y.b;
  r.a_rows_valid = first ? x.a_rows_valid : y.a_rows_valid;
  r.a_n0 = first ? x.a_n0 : y.a_n0;
  r.b_n0 = first ? x.b_n0 : y.b_n0;
  r.K = first ? x.K : y.K;
  r.brow = first ? x.brow : y.brow;
  r.bw = first ? x.bw : y.bw;
  r.stream = first ? x.stream : y.stream;
  return r;
}

// GB: the B panel gathered (GatherTile) instead of read from packed rows.
// dX tiles of 64 rows serve experts that keep few rows: when an expert has a
// single row tile, each W_e column panel is read once, so its loads stream
// past the caches (measured on the Qwen3 linear shape: dX 140 -> 120 us).
// W panels that other row tiles of the expert read again keep the default
// policy: streamed, they cost 12% at half the rows kept, and 12-24% on
// 256-row tiles.
template <class C, bool A_DIRECT, bool GB = false>
struct Stage {
  static constexpr int BAUX = (A_DIRECT && C::BM <= 64) ? kStreamAux : 0;
  using ATile = typename std::conditional<A_DIRECT, DirectTile<C::BM, C::NT>,
                                          TransTile<C::BM, C::NT>>::type;
  using BTile = typename std::conditional<GB, GatherTile<C::BN, C::NT>,
                                          TransTile<C::BN, C::NT, BAUX>>::type;
  ATile A;
  BTile B;
  int64_t lda, ldb, b_rows;
  __device__ __forceinline__ void init(int64_t la, int64_t lb, int64_t brows = 0) {
    lda = la;
    ldb = lb;
    b_rows = brows;
    A.init(la);
    B.init(lb);
  }
  __device__ __forceinline__ void load(const TileSrc& s, int k0) {
    if constexpr (A_DIRECT)
      A.load(s.a, lda, s.a_rows_valid, k0, s.K);
    else
      A.load(s.a, lda, k0, s.K, s.a_n0);
    if constexpr (GB)
      B.load(s.b, ldb, b_rows, s.b_n0);
    else
      B.load(s.b, ldb, k0, s.K, s.b_n0, s.stream);
  }
  // gathered B: the row map of the load after this one
  __device__ __forceinline__ void prefetch(const TileSrc& s, int k0) {
    if constexpr (GB) B.prefetch(s.brow, s.bw, k0, s.K);
  }
  __device__ __forceinline__ void store(uint16_t* As, uint16_t* Bs) const {
    A.store(As);
    B.store(Bs);
  }
};

struct GemmPlan {
  GemmArgs a;
  int ntm_w, ntn, nW, nX, G;  // ntn: column tiles of the dW products (and of fp32 dX)
  int ntn_x;                   // column tiles of the bf16 dX products
};

// One output tile of the stream: its K segments, k-tile counts and output.
struct Job {
  TileSrc s0, s1;
  int nk0, nk;   // k-tiles of segment 0, of both segments
  float* C;
  // split dW: tile rows from split on go to C2 (row r of the tile at C2 +
  // r * d_in); split >= the tile height: one output
  float* C2;
  int split;
  int rows, cols;  // valid output rows and columns (rows <= 0: no output)
};

// SPLIT: the dW launch writes two outputs (GemmArgs::dw_split); a template
// parameter, so that the other kernels carry none of its state.
template <class C, bool DX, bool SPLIT = false>
__device__ __forceinline__ Job make_job(const GemmPlan& P, int t) {
  const GemmArgs& a = P.a;
  Job j;
  if constexpr (!DX) {
    const int per = P.ntm_w * P.ntn;
    const int e = t / per;
    int ti, tj;
    raster(t - e * per, P.ntm_w, P.ntn, &ti, &tj);
    const int i0 = ti * C::BM, j0 = tj * C::BN;
    const int kb = ld_table(a.offsets, e);
    const int Me = max(0, min(ld_table(a.offsets, e + 1), a.max_rows) - kb);
    j.s0.a = (const char*)a.Gp + (int64_t)kb * a.d_out * 2;
    if (a.xrow) {  // gathered B: the source matrix and the expert's row map
      j.s0.b = (const char*)a.xsrc;
      j.s0.brow = a.xrow + kb;
      j.s0.bw = a.xw + kb;
    } else {
      j.s0.b = (const char*)a.Xp + (int64_t)kb * a.d_in * 2;
      j.s0.brow = nullptr;
      j.s0.bw = nullptr;
    }
    j.s0.a_rows_valid = 0; j.s0.a_n0 = i0; j.s0.b_n0 = j0;
    j.s0.K = Me;
    j.s0.stream = 0;
    j.s1 = j.s0;
    j.nk0 = j.nk = (Me + C::BK - 1) / C::BK;
    if constexpr (SPLIT) {
      // rows [0, sp) of the expert's dW in dW, rows [sp, d_out) in dW2; the
      // pointer of a part this tile does not reach is never written through
      const int sp = a.dw_split;
      j.C = a.dW + (int64_t)e * sp * a.d_in + (int64_t)i0 * a.d_in + j0;
      j.C2 = a.dW2 + (int64_t)e * (a.d_out - sp) * a.d_in + (int64_t)(i0 - sp) * a.d_in + j0;
      j.split = sp - i0;
    } else {
      j.C = a.dW + (int64_t)e * a.d_out * a.d_in + (int64_t)i0 * a.d_in + j0;
      j.C2 = j.C;
      j.split = C::BM;
    }
    j.rows = min(C::BM, a.d_out - i0);
    j.cols = min(C::BN, a.d_in - j0);
  } else {
    int mt, tn;
    const int e = dx_raster(a.mt_off, a.E, t, P.ntn_x, &mt, &tn);
    const int m0 = ld_table(a.offsets, e) + (mt - ld_table(a.mt_off, e)) * C::BM;
    const int rows = min(C::BM, min(ld_table(a.offsets, e + 1), a.max_rows) - m0);
    const int j0 = tn * C::BN;
    const int64_t lda = a.lda > 0 ? a.lda : a.d_out;
    j.s0.a = (const char*)a.Gp + m0 * lda * 2;
    j.s0.b = (const char*)a.W + (int64_t)e * a.w_stride * 2;
    j.s0.a_rows_valid = rows; j.s0.a_n0 = 0; j.s0.b_n0 = j0;
    j.s0.K = a.d_out;
    j.s0.stream = ld_table(a.mt_off, e + 1) - ld_table(a.mt_off, e) <= 1;
    j.s0.brow = nullptr;
    j.s0.bw = nullptr;
    j.s1 = j.s0;
    j.nk0 = j.nk = (a.d_out + C::BK - 1) / C::BK;
    if (a.Gp2) {  // second segment of the same shape (host-checked: d_out2 == d_out)
      j.s1.a = (const char*)a.Gp2 + m0 * lda * 2;
      j.s1.b = (const char*)a.W2 + (int64_t)e * a.w2_stride * 2;
      j.nk = 2 * j.nk0;
    }
    if (rows <= 0) j.nk = 0;
    j.C = a.dXp + (int64_t)m0 * a.d_in + j0;
    j.C2 = j.C;
    j.split = C::BM;
    j.rows = rows;
    j.cols = min(C::BN, a.d_in - j0);
  }
  return j;
}

// Tile stores are raw buffer stores through one resource per tile, bounded
// by the tile's last valid element.  Lanes outside the valid rows and columns
// take an offset past the bound, and the hardware drops their stores, so the
// stores need no per-lane branches, and each takes one offset register where
// a global store takes a 64-bit address (the 256x256 kernels: 242-245 VGPRs
// instead of 256).
constexpr int kOobOff = 0x7fff0000;  // past every tile's bound (tiles span < 1 GiB)

template <int AUX = 0>
__device__ __forceinline__ void bstore16(rsrc_t r, int off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, AUX);
}
template <int AUX = 0>
__device__ __forceinline__ void bstore8(rsrc_t r, int off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, AUX);
}

// A wave-uniform value the compiler cannot see through: offsets built from it
// are computed where the stores are, not hoisted out of the tile loop (where
// the 32 per-store offsets would take 32 live registers).
#ifdef LRM_CPU_EMU
__device__ __forceinline__ int opaque_uniform(int x) { return x; }
#else
__device__ __forceinline__ int opaque_uniform(int x) {
  asm volatile("" : "+s"(x));
  return x;
}
#endif

// Value of v in lane (l - N) mod 16 of l's 16-lane row (DPP row rotation).
template <int N>
__device__ __forceinline__ float row_rot(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x120 + N, 0xf, 0xf, false));
}

// The accumulators of a wave's 16-row block i over NF = 4 fragments
// 4J..4J+3 (16 rows x 64 columns) rearranged for row-contiguous stores:
// afterwards lane l holds row 4q + (l >> 4), columns 4 (l & 15) .. + 3 of the
// block in out[q], so each 16-lane quarter of a store covers 256 contiguous
// bytes of one row.  In the MFMA layout (lane l: row l & 15, columns
// 4 (l >> 4) .. + 3 of a fragment) a quarter stores 16 bytes into each of 16
// rows; one CU sustains about 35 GB/s of those stores against about 150 GB/s
// of 256-byte row pieces (measured on gfx950), and a tile's stores hold up
// the next tile's loads.
// Indexing (fragment f, lane bits g = l >> 4, r = l & 15 with r = 4q + a):
// swapping the fragment bits with lane bits 3..2 (DPP row rotations by 8,
// then 4 and 12) puts q in the register index and f in lane bits 3..2; a
// lane permutation exchanging lane bits 5..4 with 1..0 (ds_bpermute) then
// leaves lane (a, f, g) holding row 4q + a, columns 16 f + 4 g.
// With NF = 2 fragments 2J, 2J+1 (16 rows x 32 columns) only fragment bit 0
// and lane bit 2 are swapped: lane l then holds row 8 ((l >> 3) & 1) + 4q +
// (l >> 4), columns 4 (l & 7) .. + 3 in out[q], q < 2 (a quarter: two rows
// of 128 bytes).
template <class C, int NF>
__device__ __forceinline__ void row_major_group(const f32x4 (&acc)[C::FM][C::FN], int i, int J,
                                                f32x4 (&out)[NF]) {
  static_assert(NF == 2 || NF == 4, "fragments per group");
  const int l = lane_id();
  const bool b3 = (l >> 3) & 1, b2 = (l >> 2) & 1;
  float v[NF][4];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int k = 0; k < 4; ++k) v[f][k] = acc[i][NF * J + f][k];
  if constexpr (NF == 4) {
    // fragment bit 1 <-> lane bit 3 (lanes l and l ^ 8)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float x = v[f][k], y = v[f + 2][k];
        const float xr = row_rot<8>(x), yr = row_rot<8>(y);
        v[f][k] = b3 ? yr : x;
        v[f + 2][k] = b3 ? y : xr;
      }
  }
  // fragment bit 0 <-> lane bit 2 (lanes l and l ^ 4: l - 4 where bit 2 is
  // set, l + 4 where it is clear)
#pragma unroll
  for (int f = 0; f < NF; f += 2)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float x = v[f][k], y = v[f + 1][k];
      const float y4 = row_rot<4>(y), x12 = row_rot<12>(x);
      v[f][k] = b2 ? y4 : x;
      v[f + 1][k] = b2 ? y : x12;
    }
  // lane bits 5..4 <-> 1..0
  const int src = (((l & 3) << 4) | (l & 12) | (l >> 4)) << 2;
#pragma unroll
  for (int q = 0; q < NF; ++q)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      out[q][k] = __builtin_bit_cast(
          float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, v[q][k])));
}

// Writes a tile's accumulators (or zeros) within its valid rows and columns
// (rows <= 0: nothing is written, but every store is still issued).  Elements
// of ES bytes; lane l holds C[row = .. + (l & 15)][col = .. + (l >> 4) * 4 + 0..3].
// ROWS: the stores go out row-contiguous (row_major_group, groups of four
// fragments, or of two where a wave row holds two), non-temporal (the nt
// bit: the output is not read again by this launch, and whole lines leave
// the caches early instead of evicting operand panels); otherwise in the
// MFMA layout with the default policy (the gathering kernels, whose
// registers the rearrangement would spill; non-temporal stores of partial
// lines measured slower).  ldc < 2^20 (checked by the launcher), so a tile
// spans less than 1 GiB.
template <class C, bool BF16, bool ROWS = true>
__device__ __forceinline__ void write_tile(const f32x4 (&acc)[C::FM][C::FN], bool zero,
                                           void* out, int64_t ldc, int rows, int cols) {
  constexpr int ES = BF16 ? 2 : 4;
  const int l = lane_id(), w = threadIdx.x >> 6;
  const int wm = w / C::WGN, wn = w % C::WGN;
  const int64_t extent = (rows > 0 && cols > 0) ? ((int64_t)(rows - 1) * ldc + cols) * ES : 0;
  const rsrc_t rs = make_rsrc((const char*)out, extent);
  const int ld = opaque_uniform((int)ldc);
  if constexpr (ROWS && C::FN % 2 == 0) {
    constexpr int NF = C::FN % 4 == 0 ? 4 : 2;
    const int rl = wm * C::TM + (l >> 4) + (NF == 2 ? 8 * ((l >> 3) & 1) : 0);
    const int cl = wn * C::TN + (NF == 4 ? (l & 15) : (l & 7)) * 4;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int J = 0; J < C::FN / NF; ++J) {
        f32x4 o[NF];
        if (zero) {
#pragma unroll
          for (int q = 0; q < NF; ++q) o[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        } else {
          row_major_group<C, NF>(acc, i, J, o);
        }
#pragma unroll
        for (int q = 0; q < NF; ++q) {
          const int row = rl + i * 16 + q * 4, col = cl + J * 16 * NF;
          const int off = row < rows && col < cols ? (row * ld + col) * ES : kOobOff;
          if constexpr (BF16) {
            u32x2 v;
            v[0] = pack_bf16x2(o[q][0], o[q][1]);
            v[1] = pack_bf16x2(o[q][2], o[q][3]);
            bstore8<kStreamAux>(rs, off, v);
          } else {
            bstore16<kStreamAux>(rs, off, __builtin_bit_cast(u32x4, o[q]));
          }
        }
      }
    return;
  }
  const int row0 = wm * C::TM + (l & 15), col0 = wn * C::TN + (l >> 4) * 4;
  const int base = (row0 * ld + col0) * ES;
  const int rr = rows - row0, cc = cols - col0;
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const int bi = base + i * 16 * ld * ES;
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const bool ok = i * 16 < rr && j * 16 < cc;
      const int off = (ok ? bi : kOobOff) + j * 16 * ES;
      if constexpr (BF16) {
        u32x2 v;
        v[0] = zero ? 0u : pack_bf16x2(acc[i][j][0], acc[i][j][1]);
        v[1] = zero ? 0u : pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        bstore8(rs, off, v);
      } else {
        bstore16(rs, off, zero ? u32x4{0u, 0u, 0u, 0u} : __builtin_bit_cast(u32x4, acc[i][j]));
      }
    }
  }
}

// A finished (or zero) output tile of job j (in dW, or dW and dW2 when split,
// or dXp): dW tiles go out as bf16 when the call asks for it.  A split tile's
// waves each lie on one side of the split (it is a multiple of the wave's
// 64 rows), so each picks its output as a whole.
template <class C, bool DWB, bool SPLIT = false, bool ROWS = true>
__device__ __forceinline__ void store_tile(const GemmArgs& a, const f32x4 (&acc)[C::FM][C::FN],
                                           bool zero, const Job& j) {
  float* out = j.C;
  float* base = a.dW;
  if constexpr (SPLIT) {
    static_assert(C::TM == 64, "a wave's rows lie on one side of a split at a multiple of 64");
    const int wm = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) / C::WGN;
    const bool second = wm * C::TM >= j.split;
    out = second ? j.C2 : j.C;
    base = second ? a.dW2 : a.dW;
  }
  if constexpr (DWB)
    write_tile<C, true, ROWS>(acc, zero, reinterpret_cast<uint16_t*>(base) + (out - base),
                              a.d_in, j.rows, j.cols);
  else
    write_tile<C, false, ROWS>(acc, zero, out, a.d_in, j.rows, j.cols);
}

// MFMAs of k-granules kk..kk+3 (lane group l >> 4 takes granule kk + (l >> 4))
// on the LDS stage (Ac, Bc): B fragments once, A fragments FCH at a time.
template <class C>
__device__ __forceinline__ void mma_k32(f32x4 (&acc)[C::FM][C::FN], const uint16_t* Ac,
                                        const uint16_t* Bc, int kk) {
  const int l = lane_id(), w = threadIdx.x >> 6;
  const int wm = w / C::WGN, wn = w % C::WGN;
  bf16x8 bf[C::FN];
#pragma unroll
  for (int j = 0; j < C::FN; ++j) {
    const int col = wn * C::TN + j * 16 + (l & 15);
    bf[j] = *reinterpret_cast<const bf16x8*>(Bc + lds_off(col, 2 * (kk + (l >> 4))));
  }
#pragma unroll
  for (int i0 = 0; i0 < C::FM; i0 += C::FCH) {
    bf16x8 af[C::FCH];
#pragma unroll
    for (int i = 0; i < C::FCH; ++i) {
      const int row = wm * C::TM + (i0 + i) * 16 + (l & 15);
      af[i] = *reinterpret_cast<const bf16x8*>(Ac + lds_off(row, 2 * (kk + (l >> 4))));
    }
#pragma unroll
    for (int i = 0; i < C::FCH; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        acc[i0 + i][j] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j], af[i], acc[i0 + i][j], 0, 0, 0);
  }
}

// dW schedule.  The dW tiles, in expert order, are cut into 8 shares of equal
// cost, one per XCD, a tile of expert e costing ceil(M_e / 64) + kStoreCost:
// its k-tiles, plus its fp32 output, weighted as two k-tiles (the best of 1,
// 2, 3, 4, 8 and count-only shares measured over the Qwen3 linear, GLM-4.5
// local-32 and large SwiGLU shapes).  Inside a share the experts' runs of
// tiles are taken longest first (cost, then expert id), so that the long
// tiles of skewed experts start early and the short ones fill in at the end:
// one block per tile then is the hardware's greedy dispatch in that order (a
// longest-first schedule), and persistent blocks deal the sorted tiles in
// snake order (block b takes positions b, 2nbx - 1 - b, 2nbx + b, ...).
// Tiles inside a run keep their raster order.
//
// Heavy experts are striped: when one tile of expert e costs at least a
// quarter of a CU's ideal load (c_e * 1024 >= per * sum of c) and an expert
// has at least 8 tiles, its tiles are not part of the cut but dealt to the 8
// XCDs in 8 contiguous stripes (the i-th heavy expert's stripe s goes to XCD
// (s - i) mod 8, which spreads the longer stripes of a ragged split), and
// the other experts' tiles are cut as above.  A contiguous cut would hand
// whole shares to a heavy expert's long tiles (on the GLM-4.5 local-32
// share, 42 tiles of 141 k-tiles for 32 CUs: 1.46x the ideal in any order).
// Host model, longest CU over the ideal: 1.46 -> 1.03 (GLM-4.5 local-32
// share), 1.13 -> 1.01 (Qwen3 SwiGLU); no expert is heavy on the 65536-token
// SwiGLU and Qwen3 linear shapes (1.062 and 1.072, from longest first alone).
// Stripes cost extra operand reads: each XCD reads the panels its stripe
// needs.  With at least 8 tiles per expert, a heavy expert's cost exceeds
// 8 / 1024 of the total, so at most 128 experts are heavy.
//
// One block (k_dw_plan; 256 threads up to 1024 experts, else 1024) writes
// the schedule of a launch into the GEMM workspace after mt_off:
//   [0..8]   prefix of the share lengths in tiles
//   [9..17]  first run of each share (runs of share x: [base_x, base_{x+1}))
//   then three arrays of plan_runs(E) entries, in run order: the run's first
//   position inside its share, its expert, its first tile within the expert.
constexpr int kStoreCost = 2;
constexpr int kPlanHead = 18;
constexpr int kPlanMaxE = 4096;
constexpr int kHeavyDiv = 1024;  // heavy: c_e * kHeavyDiv >= per * sum of c
constexpr int kPlanMaxHeavy = kHeavyDiv / 8;
// runs: (share, expert) pairs of the cut (at most E + 7) plus 8 stripes per
// heavy expert
__host__ __device__ constexpr int plan_runs(int E) {
  return E + 8 + 8 * (E < kPlanMaxHeavy ? E : kPlanMaxHeavy);
}

__device__ __forceinline__ int dw_cost(const GemmArgs& a, int e) {
  const int Me = max(0, min(a.offsets[e + 1], a.max_rows) - a.offsets[e]);
  return (Me + BK - 1) / BK + kStoreCost;
}

// NT threads (E <= 4 NT: one block scan of the expert costs)
template <int NT>
// Workgroup 0 plans P0, workgroup 1 (when launched) P1: a call plans two dW
// launches at once (GemmArgs::dw_plan_next).
__global__ __launch_bounds__(NT) void k_dw_plan(GemmPlan P0, GemmPlan P1) {
  const GemmPlan& P = blockIdx.x == 0 ? P0 : P1;
  const GemmArgs& a = P.a;
  const int E = a.E, per = P.ntm_w * P.ntn, R = plan_runs(E);
  int32_t* plan = a.dw_plan;
  __shared__ int cum[kPlanMaxE + 1];  // exclusive prefix of the expert costs
  __shared__ int cst[kPlanMaxE];      // the expert costs (one read of the offsets)
  __shared__ int lds[NT / kWave + 1];
  __shared__ int lo[9], base[9], ncut[8], len[8];
  __shared__ int heavy[kPlanMaxHeavy];
  __shared__ int re[plan_runs(kPlanMaxE)], rf[plan_runs(kPlanMaxE)];
  __shared__ int rn[plan_runs(kPlanMaxE)], rc[plan_runs(kPlanMaxE)];
  const int t = threadIdx.x;
  for (int e = t; e < E; e += NT) cst[e] = dw_cost(a, e);
  __syncthreads();
  // the total cost, then the heavy experts (in expert order), then the
  // prefix of the costs with the heavy experts' left out
  block_scan_array<NT>(E, [&](int e) { return cst[e]; }, cum, lds);
  __syncthreads();
  const int64_t lim = (int64_t)per * cum[E];
  __syncthreads();
  auto is_heavy = [&](int e) {
    return per >= 8 && (int64_t)cst[e] * kHeavyDiv >= lim;
  };
  block_scan_array<NT>(E, [&](int e) { return is_heavy(e) ? 1 : 0; }, cum, lds);
  __syncthreads();
  const int nh = cum[E];
  for (int e = t; e < E; e += NT)
    if (cum[e + 1] > cum[e]) heavy[cum[e]] = e;
  if (t < 8) len[t] = 0;
  __syncthreads();
  block_scan_array<NT>(E, [&](int e) { return is_heavy(e) ? 0 : cst[e]; }, cum, lds);
  __syncthreads();
  if (t <= 8) {
    // cut start: the first tile whose start cost is >= total * t / 8 (a
    // heavy expert's tiles cost nothing here and are skipped as runs)
    int v = t == 0 ? 0 : E * per;
    if (t > 0 && t < 8) {
      if (cum[E] == 0) {
        v = 0;
      } else {
        const int64_t target = (int64_t)per * cum[E] * t / 8;
        int l = 0, h = E;  // largest e < E with per * cum[e] <= target
        while (h - l > 1) {
          const int m = (l + h) >> 1;
          if ((int64_t)per * cum[m] <= target) l = m; else h = m;
        }
        const int c = cum[l + 1] - cum[l];  // > 0: per * cum[l + 1] > target
        const int64_t j = (target - (int64_t)per * cum[l] + c - 1) / c;
        v = l * per + (int)min<int64_t>(j, per);
      }
    }
    lo[t] = v;
  }
  __syncthreads();
  if (t == 0) {
    int n = 0;
    for (int x = 0; x < 8; ++x) {
      base[x] = n;
      ncut[x] = lo[x + 1] > lo[x] ? (lo[x + 1] - 1) / per - lo[x] / per + 1 : 0;
      n += ncut[x] + nh;
    }
    base[8] = n;
  }
  __syncthreads();
  const int nr = base[8];
  // each share's runs: those of the cut in expert order (a heavy expert's
  // with no tiles), then one stripe of every heavy expert
  for (int r = t; r < nr; r += NT) {
    int x = 0;
    while (base[x + 1] <= r) ++x;
    const int i = r - base[x];
    if (i < ncut[x]) {
      const int e = lo[x] / per + i;
      const int a0 = max(lo[x], e * per), a1 = min(lo[x + 1], (e + 1) * per);
      const int c = cum[e + 1] - cum[e];  // 0: a heavy expert
      re[r] = e;
      rf[r] = a0 - e * per;
      rn[r] = c > 0 ? a1 - a0 : 0;
      rc[r] = c;
    } else {
      const int k = i - ncut[x];
      const int e = heavy[k];
      const int sx = (x + k) & 7;
      const int f0 = per * sx / 8, f1 = per * (sx + 1) / 8;
      re[r] = e;
      rf[r] = f0;
      rn[r] = f1 - f0;
      rc[r] = cst[e];
    }
    atomicAdd(&len[x], rn[r]);
  }
  __syncthreads();
  if (t == 0) {
    int n = 0;
    for (int x = 0; x < 8; ++x) {
      plan[x] = n;
      n += len[x];
      plan[9 + x] = base[x];
    }
    plan[8] = n;
    plan[17] = base[8];
  }
  // rank of each run inside its share (cost descending, then run order) and
  // its first position: the tiles of the runs ranked before it
  for (int r = t; r < nr; r += NT) {
    int x = 0;
    while (base[x + 1] <= r) ++x;
    int rank = 0, pos = 0;
    for (int q = base[x]; q < base[x + 1]; ++q) {
      if (rc[q] > rc[r] || (rc[q] == rc[r] && q < r)) {
        ++rank;
        pos += rn[q];
      }
    }
    plan[kPlanHead + base[x] + rank] = pos;
    plan[kPlanHead + R + base[x] + rank] = re[r];
    plan[kPlanHead + 2 * R + base[x] + rank] = rf[r];
  }
}

// The tiles one block runs, in order: tile at(k) of the launch's list, or -1
// past the block's part of its XCD share.  dX: the share's tiles lo + b,
// lo + b + nbx, ...  dW: the scheduled order above (runs scanned forward:
// a block's positions only grow).
struct TileSeq {
  const int32_t* pre;  // dW: run starts of the share; experts at +R, first tiles at +2R
  int R, lo, len, b, nbx, per, nrun, s;
  __device__ __forceinline__ int at(int k) {
    if (!pre) {
      const int i = b + k * nbx;
      return i < len ? lo + i : -1;
    }
    const int p = k * nbx + ((k & 1) ? nbx - 1 - b : b);
    if (p >= len) return -1;
    while (s + 1 < nrun && ld_table(pre, s + 1) <= p) ++s;
    return ld_table(pre, R + s) * per + ld_table(pre, 2 * R + s) + (p - ld_table(pre, s));
  }
};

template <bool DX>
__device__ __forceinline__ TileSeq tile_seq(const GemmPlan& P) {
  const GemmArgs& a = P.a;
  const int x = blockIdx.x & 7;
  TileSeq q;
  q.b = blockIdx.x >> 3;
  q.nbx = gridDim.x >> 3;
  q.per = P.ntm_w * P.ntn;
  q.s = 0;
  q.nrun = 0;
  q.R = 0;
  q.pre = nullptr;
  if constexpr (DX) {
    // every dX tile runs K = d_out: equal shares of the tile count
    const int n = ld_table(a.mt_off, a.E) * P.ntn_x;
    q.lo = (int)((int64_t)n * x / 8);
    q.len = (int)((int64_t)n * (x + 1) / 8) - q.lo;
  } else {
    const int32_t* pl = a.dw_plan;
    q.R = plan_runs(a.E);
    q.lo = ld_table(pl, x);
    q.len = ld_table(pl, x + 1) - q.lo;
    const int b0 = ld_table(pl, 9 + x);
    q.nrun = ld_table(pl, 10 + x) - b0;
    q.pre = pl + kPlanHead + b0;
  }
  return q;
}

// Persistent tile stream.  Each XCD takes a contiguous eighth of the tile list
// (consecutive tiles share operand panels in its L2) and its blocks take the
// tiles of that range in turn (dW: in the scheduled order, TileSeq).  A block runs the k-tiles of all its tiles as
// one stream: two LDS stages, the registers of the next k-tile stored into the
// idle stage while the MFMAs consume the current one, global loads two k-tiles
// ahead, one barrier per k-tile.  The loads of a tile's first k-tiles are thus
// in flight while the previous tile's outputs are written.  A tile with no
// k-tiles (an expert that kept no rows) writes zeros.
template <class C, bool DX, bool DWB, bool GB = false, bool SPLIT = false>
__device__ __forceinline__ void gemm_stream(const GemmPlan& P) {
  __shared__ __attribute__((aligned(16))) uint16_t As[C::STAGES * C::BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[C::STAGES * C::BN * BK];
  const GemmArgs& a = P.a;
  // the block's tiles, in order (compute cursor sc, load cursor sl)
  TileSeq sc = tile_seq<DX>(P);
  int kcn = 0;
  int tc = sc.at(0);

  f32x4 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // compute cursor: tile tc (job jc), k-tile kc; zero tiles are written as met
  Job jc;
  for (; tc >= 0; tc = sc.at(++kcn)) {
    jc = make_job<C, DX, SPLIT>(P, tc);
    if (jc.nk > 0) break;
    if (jc.rows > 0) store_tile<C, DWB, SPLIT, !GB>(a, acc, true, jc);
  }
  if (tc < 0) return;

  Stage<C, DX, GB> st;
  if constexpr (GB)
    st.init(a.lda > 0 ? a.lda : a.d_out, a.ldxs, a.xsrc_rows);
  else
    st.init(a.lda > 0 ? a.lda : a.d_out, a.d_in);
  // load cursor: tile tl (job jl), k-tile kl, two k-tiles ahead of the compute
  TileSeq sl = sc;
  int kln = kcn;
  int tl = tc, kl = 0;
  Job jl = jc;
  if constexpr (GB) st.prefetch(jl.s0, 0);  // the row map of the first load
#define LRM_ISSUE_LOAD()                                                        \
  if (tl >= 0) {                                                                \
    const bool first = kl < jl.nk0;                                             \
    st.load(pick_seg(jl.s0, jl.s1, first), (first ? kl : kl - jl.nk0) * BK);   \
    if (++kl == jl.nk) {                                                        \
      kl = 0;                                                                   \
      for (tl = sl.at(++kln); tl >= 0; tl = sl.at(++kln)) {                     \
        jl = make_job<C, DX, SPLIT>(P, tl);                                            \
        if (jl.nk > 0) break;                                                   \
      }                                                                         \
    }                                                                           \
    if (GB && tl >= 0) {                                                        \
      const bool f2 = kl < jl.nk0;                                              \
      st.prefetch(pick_seg(jl.s0, jl.s1, f2), (f2 ? kl : kl - jl.nk0) * BK);   \
    }                                                                           \
  }
  // With two LDS stages the loads of k-tile i+2 are issued as soon as k-tile
  // i+1 has left the registers for LDS, in the middle of k-tile i's MFMAs,
  // which gives them a whole k-tile of MFMAs to arrive (issued after the
  // MFMAs, they get half of one).
  constexpr bool kEarlyLoad = C::STAGES == 2;
  LRM_ISSUE_LOAD();
  st.store(As, Bs);
  LRM_ISSUE_LOAD();
  __syncthreads();
  int it = 0;
  // One k-tile: MFMAs on the current stage, the next k-tile's registers into
  // the idle stage, the load two k-tiles ahead.
#define LRM_KSTEP()                                                             \
  {                                                                             \
    const int cur = C::STAGES == 2 ? (it & 1) : 0;                              \
    const uint16_t* Ac = As + cur * (C::BM * BK);                               \
    const uint16_t* Bc = Bs + cur * (C::BN * BK);                               \
    mma_k32<C>(acc, Ac, Bc, 0);                                                 \
    if constexpr (C::STAGES == 2)                                               \
      st.store(As + (cur ^ 1) * (C::BM * BK), Bs + (cur ^ 1) * (C::BN * BK));   \
    if constexpr (kEarlyLoad) LRM_ISSUE_LOAD();                                 \
    mma_k32<C>(acc, Ac, Bc, 4);                                                 \
    if constexpr (C::STAGES == 1) {                                             \
      __syncthreads();                                                          \
      st.store(As, Bs);                                                         \
    }                                                                           \
    if constexpr (!kEarlyLoad) LRM_ISSUE_LOAD();                                \
    ++it;                                                                       \
  }
  int kc = 0;
  for (;;) {
    LRM_KSTEP();
    if (++kc == jc.nk) {
      store_tile<C, DWB, SPLIT, !GB>(a, acc, false, jc);
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      kc = 0;
      for (tc = sc.at(++kcn); tc >= 0; tc = sc.at(++kcn)) {
        jc = make_job<C, DX, SPLIT>(P, tc);
        if (jc.nk > 0) break;
        if (jc.rows > 0) store_tile<C, DWB, SPLIT, !GB>(a, acc, true, jc);
      }
      if (tc < 0) break;
    }
    __syncthreads();
  }
#undef LRM_KSTEP
#undef LRM_ISSUE_LOAD
}

template <class C, bool DX>
__global__ __launch_bounds__(C::NT, C::WPE) void k_gemm_stream(GemmPlan P) {
  gemm_stream<C, DX, false>(P);
}

// dW products stored as bf16 (a separate kernel: the fp32 kernels keep their
// code and registers)
template <class C>
__global__ __launch_bounds__(C::NT, C::WPE) void k_gemm_stream_dwbf16(GemmPlan P) {
  gemm_stream<C, false, true>(P);
}

// dW products split over two outputs (GemmArgs::dw_split), fp32 or bf16 dW
template <class C, bool DWB>
__global__ __launch_bounds__(C::NT, C::WPE) void k_gemm_stream_split(GemmPlan P) {
  gemm_stream<C, false, DWB, false, true>(P);
}

// dW products with the B panel gathered from its source rows (fp32 or bf16 dW)
template <class C, bool DWB>
__global__ __launch_bounds__(C::NT, C::WPE) void k_gemm_stream_gather(GemmPlan P) {
  gemm_stream<C, false, DWB, true>(P);
}

// ------------------------------------------------------------ LDS-DMA stream
//
// An alternative to the register path for 256x256 tiles whose operand rows
// start on 16-byte boundaries (and, for dX, whose K is a whole number of
// k-tiles), selected with LRM_GEMM_DMA (see dma_choice).  Operand tiles go from
// global memory straight into LDS: buffer loads with the LDS-destination flag,
// 16 bytes per lane, each instruction filling 1 KB of LDS (lane p at byte
// 16p).  No staging registers, register transposes or LDS stores; the
// registers left over go to fragments.  k-strided operands (dW's A and B,
// dX's B) stay in LDS as they lie in memory, [k][n] with n contiguous, and
// are read with ds_read_b64_tr_b16: within each 16-lane group, output lane j
// element r is element j % 4 of the 8 bytes addressed by lane 4r + j / 4
// (measured), so lanes addressing 4 k-rows x 16 columns receive one column's
// 4 consecutive k each; two such reads make an MFMA operand fragment.  dX's A
// (k contiguous) keeps the [m][k] layout of the register path.
//
// STAGES LDS stages of BK k each; loads run STAGES - 1 k-tiles ahead of the
// MFMAs.  A k-tile is consumed after a wait for the wave's own loads of it
// (the vector memory counter retires loads and stores in issue order, so the
// wait names how many younger instructions may still be outstanding) and a
// barrier; the barrier also frees the stage consumed one k-tile earlier, which
// receives the next loads.
template <int BK_, int STAGES_>
struct DmaCfg {
  static constexpr int BM = 256, BN = 256, BK = BK_, STAGES = STAGES_;
  static constexpr int MINB = 1, WGM = 4, WGN = 2, NW = 8, NT = 512, WPE = 2;
  static constexpr int TM = 64, TN = 128, FM = 4, FN = 8, FCH = 4;
  static constexpr int NQ = BK / 16;  // LDS-DMA instructions per operand, wave and k-tile
  static constexpr int NSTORE = FM * FN;  // buffer stores per wave and output tile
  static_assert(BK == 32 || BK == 64, "k-tile");
  static_assert(2 * NQ * (STAGES - 1) + NSTORE <= 63, "vector memory counter range");
};

#ifdef LRM_CPU_EMU
typedef void* lds_vptr;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef s16x4* lds_s16x4;
#else
typedef __attribute__((address_space(3))) void* lds_vptr;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4;
#endif

// 16 bytes per lane from r at byte voff into LDS at lds + 16 * lane (lds is
// wave-uniform); past the bound the lane writes zeros (measured).  Written
// as inline asm so that the compiler, which does not track these loads, does
// not wait for every one in flight before each LDS read: the kernel orders
// them itself (dma_barrier).  The LDS address goes in M0 as an input operand.
#ifdef LRM_CPU_EMU
typedef rsrc_t dma_rsrc;
__device__ __forceinline__ dma_rsrc make_dma_rsrc(const char* base, int64_t nbytes) {
  return make_rsrc(base, nbytes);
}
__device__ __forceinline__ void dma16(dma_rsrc r, uint16_t* lds, int voff) {
  const u32x4 v = bload(r, voff);
  std::memcpy(reinterpret_cast<char*>(lds) + 16 * lane_id(), &v, 16);
}
#else
typedef u32x4 dma_rsrc;  // buffer resource words: base, bound, raw access
__device__ __forceinline__ dma_rsrc make_dma_rsrc(const char* base, int64_t nbytes) {
  const int n = nbytes <= 0 ? 0 : (nbytes > 0x7ffffff0ll ? 0x7ffffff0 : (int)nbytes);
  const uint64_t b = (uint64_t)(uintptr_t)base;
  return dma_rsrc{(uint32_t)b, (uint32_t)(b >> 32) & 0xffffu, (uint32_t)n, (uint32_t)kRsrcWord3};
}
__device__ __forceinline__ void dma16(dma_rsrc r, uint16_t* lds, int voff) {
  const uint32_t la = (uint32_t)(uintptr_t)(lds_vptr)lds;
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "{m0}"(la)
               : "memory");
}
#endif

// [k][n] LDS tile of 256 columns (512-byte rows) in 32-byte segments; segment
// c of row k sits at c ^ trh(k).  A transposed read by 16 lanes covers one
// segment of 4 consecutive rows; two 16-lane groups read rows 8 (or 16) apart.
// trh gives those 8 row-segments distinct positions modulo 8, i.e. distinct
// 32-byte bank slots of the 256-byte bank cycle.
__device__ __forceinline__ int trh(int k) {
  return (k & 3) | (((k >> 3) ^ (k >> 4)) & 1) << 2;
}
// [m][k] rows of 32 k (64 bytes): granule G of row r at G ^ swz32(r).  With
// the four 16-lane passes of a ds_read_b128 (lanes 0-3, 12-15, 20-23, 24-27;
// 4-7, 8-11, 16-19, 28-31; the same +32) every pass hits 16 distinct granule
// slots of the bank cycle.
__device__ __forceinline__ int swz32(int r) { return (4 - ((r >> 2) & 3)) & 3; }

__device__ __forceinline__ s16x4 ldtr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)const_cast<uint16_t*>(p));
}
// fragment of 16 columns, k rows kr..kr+3 and kr+4..kr+7 (p at row kr)
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* p) {
  const s16x4 lo = ldtr(p), hi = ldtr(p + 4 * 256);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Per-lane byte offsets of a wave's LDS-DMA granules (fixed for the launch:
// the operand's leading dimension does not change) and the k-tile loads.
template <class C, bool DX>
struct DmaStage {
  static constexpr int NQ = C::NQ;
  int offa[NQ], offb[NQ];
  int w;
  int64_t lda, ldb;
  // granule p of 1 KB block b of a [k][256] tile (rows 2b, 2b + 1)
  __device__ __forceinline__ static int kstr_off(int b, int p, int64_t ld) {
    const int k = 2 * b + (p >> 5), s = p & 31;
    const int c = (s >> 1) ^ trh(k);
    return (int)(k * ld * 2) + c * 32 + (s & 1) * 16;
  }
  // granule p of 1 KB block b of a [256][BK] tile
  __device__ __forceinline__ static int kcont_off(int b, int p, int64_t ld) {
    if constexpr (C::BK == 64) {
      const int r = 8 * b + (p >> 3);
      return (int)(r * ld * 2) + (((p & 7) ^ lds_swz(r)) << 4);
    } else {
      const int r = 16 * b + (p >> 2);
      return (int)(r * ld * 2) + (((p & 3) ^ swz32(r)) << 4);
    }
  }
  __device__ __forceinline__ void init(int64_t la, int64_t lb) {
    lda = la;
    ldb = lb;
    w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int p = lane_id();
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int b = w * NQ + q;
      offa[q] = DX ? kcont_off(b, p, la) : kstr_off(b, p, la);
      offb[q] = kstr_off(b, p, lb);
    }
  }
  // k-tile [k0, k0 + BK) of segment s into the stage (As, Bs).  Bounds as in
  // the register path: rows past the expert's block (dX's A) or past K (the
  // k-strided panels) read zeros; columns past the operand's width read the
  // next row, which only reaches output columns that are never stored.
  __device__ __forceinline__ void load(const TileSrc& s, int k0, uint16_t* As, uint16_t* Bs) const {
    const dma_rsrc ra =
        DX ? make_dma_rsrc(s.a + (int64_t)k0 * 2, (int64_t)s.a_rows_valid * lda * 2 - k0 * 2)
           : make_dma_rsrc(s.a + ((int64_t)k0 * lda + s.a_n0) * 2,
                           (int64_t)(s.K - k0) * lda * 2 - (int64_t)s.a_n0 * 2);
    const dma_rsrc rb = make_dma_rsrc(s.b + ((int64_t)k0 * ldb + s.b_n0) * 2,
                                      (int64_t)(s.K - k0) * ldb * 2 - (int64_t)s.b_n0 * 2);
#pragma unroll
    for (int q = 0; q < NQ; ++q) dma16(ra, As + (w * NQ + q) * 512, offa[q]);
#pragma unroll
    for (int q = 0; q < NQ; ++q) dma16(rb, Bs + (w * NQ + q) * 512, offb[q]);
  }
};

// Per-lane LDS element offsets of a wave's fragments at k = 0 of a stage.
template <class C, bool DX>
struct DmaFrag {
  int tb[C::FN];   // B fragment j ([k][n])
  int ta[C::FM];   // A fragment i ([k][m]; dX: [m][k], k 0..31)
  int ta1[C::FM];  // dX with BK 64: A fragment i, k 32..63
  __device__ __forceinline__ void init() {
    const int l = lane_id(), w = threadIdx.x >> 6;
    const int wm = w / C::WGN, wn = w % C::WGN;
    const int g = l >> 4, i = l & 15;
    const int kr = 8 * g + (i >> 2);  // first k row of this lane's transposed reads
    const int t = trh(kr);            // the same for rows kr + 32 and kr + 4
    const int base = kr * 256 + 4 * (i & 3);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) tb[j] = base + (((wn * (C::TN / 16) + j) ^ t) << 4);
#pragma unroll
    for (int f = 0; f < C::FM; ++f) {
      if constexpr (DX) {
        const int row = wm * C::TM + f * 16 + i;
        if constexpr (C::BK == 64) {
          ta[f] = lds_off(row, 2 * g);
          ta1[f] = lds_off(row, 2 * (4 + g));
        } else {
          ta[f] = row * 32 + ((g ^ swz32(row)) << 3);
          ta1[f] = ta[f];
        }
      } else {
        ta[f] = base + (((wm * (C::TM / 16) + f) ^ t) << 4);
        ta1[f] = ta[f];
      }
    }
  }
};

// The MFMAs of k 32h..32h+31 of a stage.
template <class C, bool DX>
__device__ __forceinline__ void mma_dma(f32x4 (&acc)[C::FM][C::FN], const uint16_t* As,
                                        const uint16_t* Bs, const DmaFrag<C, DX>& f, int h) {
  bf16x8 bf[C::FN], af[C::FM];
#pragma unroll
  for (int j = 0; j < C::FN; ++j) bf[j] = tr_frag(Bs + h * 32 * 256 + f.tb[j]);
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    if constexpr (DX)
      af[i] = *reinterpret_cast<const bf16x8*>(As + (h ? f.ta1[i] : f.ta[i]));
    else
      af[i] = tr_frag(As + h * 32 * 256 + f.ta[i]);
  }
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (expcnt not waited on)
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
// Wait until at most n vector memory instructions of this wave are
// outstanding, then the block barrier.  n is rounded down to a value of the
// ladder {0, L, 2L, NSTORE, NSTORE + L, NSTORE + 2L, 60} (L = 2 NQ, the loads
// of one k-tile): the counts that occur are the loads of up to two younger
// k-tiles, plus one output tile's stores; anything past that waits for 60.
// The empty asm statements keep the compiler from moving LDS accesses across.
template <class C>
__device__ __forceinline__ void dma_barrier(int n) {
  constexpr int L = 2 * C::NQ, T = C::NSTORE;
  static_assert(T + 2 * L <= 60, "ladder");
  asm volatile("" ::: "memory");
  if (n >= 60) wait_vm<60>();
  else if (n >= T + 2 * L) wait_vm<T + 2 * L>();
  else if (n >= T + L) wait_vm<T + L>();
  else if (n >= T) wait_vm<T>();
  else if (n >= 2 * L) wait_vm<2 * L>();
  else if (n >= L) wait_vm<L>();
  else wait_vm<0>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <class C, bool DX, bool DWB>
__device__ __forceinline__ void gemm_dma(const GemmPlan& P) {
  constexpr int S = C::STAGES;
  constexpr int SA = C::BM * C::BK, SS = (C::BM + C::BN) * C::BK;  // elements
  __shared__ __attribute__((aligned(1024))) uint16_t L[S * SS];
  const GemmArgs& a = P.a;
  TileSeq sc = tile_seq<DX>(P);
  int kcn = 0;
  int tc = sc.at(0);

  f32x4 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Tiles with no k-tiles (experts that kept no rows) are written from acc,
  // which is zero wherever they are met (stored as constants, the zeros of
  // the fp32 stores end up spilled as scalar registers).
  Job jc;
  for (; tc >= 0; tc = sc.at(++kcn)) {
    jc = make_job<C, DX>(P, tc);
    if (jc.nk > 0) break;
    if (jc.rows > 0) store_tile<C, DWB>(a, acc, false, jc);
  }
  if (tc < 0) return;

  DmaStage<C, DX> st;
  st.init(a.lda > 0 ? a.lda : a.d_out, a.d_in);
  DmaFrag<C, DX> fr;
  fr.init();
  // vm: vector memory instructions this wave has issued since the first load
  // (every wave issues the same ones); mk[s]: vm just after the loads of the
  // s-th oldest k-tile in flight
  int vm = 0, mk[S];
  TileSeq sl = sc;
  int kln = kcn;
  int tl = tc, kl = 0, nxt = 0;
  Job jl = jc;
  // the next k-tile of the stream (if any) into stage nxt, its mark in mk[slot]
  auto issue = [&](int slot) {
    if (tl >= 0) {
      const bool first = kl < jl.nk0;
      uint16_t* dst = L + nxt * SS;
      st.load(pick_seg(jl.s0, jl.s1, first), (first ? kl : kl - jl.nk0) * C::BK, dst, dst + SA);
      vm += 2 * C::NQ;
      if (++kl == jl.nk) {
        kl = 0;
        for (tl = sl.at(++kln); tl >= 0; tl = sl.at(++kln)) {
          jl = make_job<C, DX>(P, tl);
          if (jl.nk > 0) break;
        }
      }
    }
    mk[slot] = vm;
    nxt = nxt + 1 == S ? 0 : nxt + 1;
  };
#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(s);
  int cur = 0, kc = 0;
  for (;;) {
    dma_barrier<C>(vm - mk[0]);
    issue(S - 1);
    const uint16_t* Ac = L + cur * SS;
#pragma unroll
    for (int h = 0; h < C::BK / 32; ++h) mma_dma<C, DX>(acc, Ac, Ac + SA, fr, h);
    cur = cur + 1 == S ? 0 : cur + 1;
#pragma unroll
    for (int s = 0; s < S - 1; ++s) mk[s] = mk[s + 1];
    if (++kc == jc.nk) {
      // the finished tile, then any tiles with no k-tiles up to the next one
      // that has some (one store site: a second one costs scalar spills)
      bool done = false;
      for (;;) {
        if (jc.rows > 0) {
          store_tile<C, DWB>(a, acc, false, jc);
          vm += C::NSTORE;
        }
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        tc = sc.at(++kcn);
        if (tc < 0) {
          done = true;
          break;
        }
        jc = make_job<C, DX>(P, tc);
        if (jc.nk > 0) break;
      }
      if (done) break;
      kc = 0;
    }
  }
}

template <class C, bool DX, bool DWB>
__global__ __launch_bounds__(C::NT, C::WPE) void k_gemm_dma(GemmPlan P) {
  gemm_dma<C, DX, DWB>(P);
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
    const int kb = ld_table(a.offsets, e);
    const int Me = max(0, min(ld_table(a.offsets, e + 1), a.max_rows) - kb);
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

// Tile configurations of the bf16 kernel.
using CfgS = TileCfg<128, 128, 2, 2, 2>;  // 4 waves of 64x64
using CfgM = TileCfg<256, 128, 4, 2>;   // 8 waves of 64x64
using CfgL = TileCfg<256, 256, 4, 2>;   // 8 waves of 64x128
using CfgXS = TileCfg<64, 256, 1, 8, 2>;  // 8 waves of 64x32 (dX of small experts)

// Plan the combined tile list (dW tiles tmw x tn, dX tiles tmx x tn) and build
// the dX row-tile prefix on the device.
static hipError_t plan_tiles(const GemmArgs& a, int tmw, int tnw, int tmx, int tnx, GemmPlan* P,
                             hipStream_t s) {
  P->a = a;
  P->ntn = (a.d_in + tnw - 1) / tnw;
  P->ntn_x = (a.d_in + tnx - 1) / tnx;
  P->ntm_w = (a.d_out + tmw - 1) / tmw;
  P->nW = a.dW ? a.E * P->ntm_w * P->ntn : 0;
  P->nX = (a.dXp && a.max_rows > 0) ? ((a.max_rows + tmx - 1) / tmx + a.E) * P->ntn_x : 0;
  if (P->nX > 0 && !a.mt_ready) {
    hipError_t err = launch_tile_plan(a.E, tmx, a.offsets, a.mt_off, s);
    if (err != hipSuccess) return err;
  }
  const int64_t total = (int64_t)P->nW + P->nX;
  if (total > (1ll << 30)) return hipErrorInvalidValue;
  P->G = (int)((total + 7) & ~7ll);
  return hipSuccess;
}

// Resident blocks of a GEMM kernel on the current device, cached for the
// first 16 devices (concurrent callers may both compute it; they store the
// same value).
template <auto Kern, int NTH>
static int grid_cap_of() {
  static std::atomic<int> cap[16];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 16) {
    const int c = cap[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0, occ = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, Kern, NTH, 0) != hipSuccess || occ <= 0)
    occ = 1;
  const int c = cus * occ;
  if (dev < 16) cap[dev].store(c, std::memory_order_relaxed);
  return c;
}

template <class C, bool DX, bool DWB = false>
static int stream_grid_cap() {
  if constexpr (DWB)
    return grid_cap_of<k_gemm_stream_dwbf16<C>, C::NT>();
  else
    return grid_cap_of<k_gemm_stream<C, DX>, C::NT>();
}

// per_tile: one block per tile (a multiple of 8 blocks), the hardware handing
// tiles to CUs as they free up; otherwise at most one resident round of
// persistent blocks, each running its share of the tiles as one stream.
template <class C, bool DX>
static hipError_t launch_stream(const GemmPlan& P, int ntiles_max, hipStream_t s,
                                bool per_tile) {
  if (ntiles_max <= 0) return hipSuccess;
  const int64_t want = ((int64_t)ntiles_max + 7) & ~7ll;
  if constexpr (!DX) {
    if (P.a.dw_split > 0) {
      // the split dW kernels (their residency is that of the plain ones)
      const int G = per_tile ? (int)want
                             : (int)std::min<int64_t>(
                                   want, std::max(8, stream_grid_cap<C, false>() & ~7));
      if (P.a.dw_bf16)
        LRM_LAUNCH(G, C::NT, 0, s, k_gemm_stream_split<C, true>)(P);
      else
        LRM_LAUNCH(G, C::NT, 0, s, k_gemm_stream_split<C, false>)(P);
      return hipGetLastError();
    }
    if (P.a.xrow) {
      // the gathering dW kernels (their residency is that of the plain ones)
      const int G = per_tile ? (int)want
                             : (int)std::min<int64_t>(
                                   want, std::max(8, stream_grid_cap<C, false>() & ~7));
      if (P.a.dw_bf16)
        LRM_LAUNCH(G, C::NT, 0, s, k_gemm_stream_gather<C, true>)(P);
      else
        LRM_LAUNCH(G, C::NT, 0, s, k_gemm_stream_gather<C, false>)(P);
      return hipGetLastError();
    }
    if (P.a.dw_bf16) {
      const int G = per_tile ? (int)want
                             : (int)std::min<int64_t>(
                                   want, std::max(8, stream_grid_cap<C, false, true>() & ~7));
      LRM_LAUNCH(G, C::NT, 0, s, k_gemm_stream_dwbf16<C>)(P);
      return hipGetLastError();
    }
  }
  const int G = per_tile
                    ? (int)want
                    : (int)std::min<int64_t>(want, std::max(8, stream_grid_cap<C, DX>() & ~7));
  LRM_LAUNCH(G, C::NT, 0, s, k_gemm_stream<C, DX>)(P);
  return hipGetLastError();
}

// The LDS-DMA kernels (256x256 tiles), opt-in: LRM_GEMM_DMA=2 (k-tiles of
// 64, two stages) or 4 (k-tiles of 32, four stages).  Measured on the
// 65536-token SwiGLU shapes they match the register path (dW, four stages)
// or trail it by 3-15% (dX): both wait on L2 for about 43% of the wave
// cycles, bound by the requests a CU may have in flight (its L1 stalls on
// pending L2 data most of the time), which direct loads do not change.
using CfgD = DmaCfg<64, 2>;
using CfgD4 = DmaCfg<32, 4>;

static int dma_choice() {
  const char* env = getenv("LRM_GEMM_DMA");
  if (env && env[0] == '2') return 2;
  if (env && env[0] == '4') return 4;
  return 0;
}

// Operand rows and bases on 16-byte boundaries; dX: K a whole number of
// k-tiles (the k-contiguous A panel has no per-lane k bound); dW: packed B
// rows (the gathering loaders scale rows in registers).
template <class C>
static bool dma_ok(const GemmArgs& a, bool dx) {
  auto al = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  if (a.d_in % 8 || a.d_out % 8 || a.lda % 8 || !al(a.Gp)) return false;
  if (!dx) return !a.xrow && al(a.Xp);
  if (a.d_out % C::BK || !al(a.W) || a.w_stride % 8) return false;
  return !a.Gp2 || (al(a.Gp2) && al(a.W2) && a.w2_stride % 8 == 0);
}

template <class C, bool DX>
static hipError_t launch_dma(const GemmPlan& P, int ntiles_max, hipStream_t s, bool per_tile) {
  if (ntiles_max <= 0) return hipSuccess;
  const int64_t want = ((int64_t)ntiles_max + 7) & ~7ll;
  const bool dwb = !DX && P.a.dw_bf16;
  const int cap = DX    ? grid_cap_of<k_gemm_dma<C, true, false>, C::NT>()
                  : dwb ? grid_cap_of<k_gemm_dma<C, false, true>, C::NT>()
                        : grid_cap_of<k_gemm_dma<C, false, false>, C::NT>();
  const int G = per_tile ? (int)want : (int)std::min<int64_t>(want, std::max(8, cap & ~7));
  if (DX)
    LRM_LAUNCH(G, C::NT, 0, s, k_gemm_dma<C, true, false>)(P);
  else if (dwb)
    LRM_LAUNCH(G, C::NT, 0, s, k_gemm_dma<C, false, true>)(P);
  else
    LRM_LAUNCH(G, C::NT, 0, s, k_gemm_dma<C, false, false>)(P);
  return hipGetLastError();
}

// One product's launch: the LDS-DMA kernel for 256x256 tiles when the
// operands allow it, the register-path stream otherwise.
template <class C, bool DX>
static hipError_t launch_product(const GemmPlan& P, int ntiles_max, hipStream_t s,
                                 bool per_tile) {
  if constexpr (std::is_same<C, CfgL>::value) {
    const int d = P.a.dw_split > 0 ? 0 : dma_choice();  // the DMA kernels write one dW
    if (d == 2 && dma_ok<CfgD>(P.a, DX)) return launch_dma<CfgD, DX>(P, ntiles_max, s, per_tile);
    if (d == 4 && dma_ok<CfgD4>(P.a, DX))
      return launch_dma<CfgD4, DX>(P, ntiles_max, s, per_tile);
  }
  return launch_stream<C, DX>(P, ntiles_max, s, per_tile);
}

int64_t gemm_workspace_ints(int E) {
  return (int64_t)E + 1 + kPlanHead + 3 * (int64_t)plan_runs(E);
}

// The fields of a GemmPlan that k_dw_plan reads, for the dW launch of b (bf16
// kernels, its tile configuration): false if b has no scheduled dW launch.
static bool dw_plan_of(const GemmArgs& b, GemmPlan* Q) {
  if (gemm_dw_tiles_per_expert(b) <= 0) return false;
  int bm = CfgS::BM, bn = CfgS::BN;
  switch (gemm_tile_choice(b)) {
    case 3:
    case 2: bm = CfgL::BM; bn = CfgL::BN; break;
    case 1: bm = CfgM::BM; bn = CfgM::BN; break;
    default: break;
  }
  *Q = GemmPlan{};
  Q->a = b;
  Q->ntm_w = (b.d_out + bm - 1) / bm;
  Q->ntn = (b.d_in + bn - 1) / bn;
  Q->nW = b.E * Q->ntm_w * Q->ntn;
  Q->a.dw_plan = b.mt_off + b.E + 1;
  return true;
}

template <class CW, class CX>
static hipError_t launch_bf16(const GemmArgs& a, hipStream_t s) {
  GemmPlan P{};
  hipError_t err = plan_tiles(a, CW::BM, CW::BN, CX::BM, CX::BN, &P, s);
  if (err != hipSuccess) return err;
  if (P.nW > 0) {
    P.a.dw_plan = a.mt_off + a.E + 1;
    if (!a.dw_plan_ready) {
      // the next launch's schedule in the same launch, by a second workgroup
      GemmPlan P2 = P;
      const GemmArgs* nx = a.dw_plan_next;
      const int nb = nx && nx->E == a.E && nx->mt_off && dw_plan_of(*nx, &P2) ? 2 : 1;
      if (a.E <= 4 * 256)
        LRM_LAUNCH(nb, 256, 0, s, k_dw_plan<256>)(P, P2);
      else
        LRM_LAUNCH(nb, 1024, 0, s, k_dw_plan<1024>)(P, P2);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
  }
  // With many rows per expert (256x256 tiles for both products, MFMA-bound)
  // the k-tile counts of dW tiles follow the expert sizes, which are skewed.
  // Each XCD still takes its share of equal cost, but with one block per tile
  // (up to 16 resident rounds) the hardware balances the tiles inside a share
  // as CUs free up, where persistent blocks would each hold a fixed slice.
  // Measured: Qwen3 SwiGLU shape -5.7%, GLM-4.5 local share even, and the
  // 65536-token shape (48 rounds) +2.4%, hence the bound.  With few rows per
  // expert the persistent stream keeps its one-k-tile tiles fed.
  const int rounds = std::max(P.nW, P.nX) / std::max(1, stream_grid_cap<CW, false>());
  const bool per_tile = gemm_tile_choice(a) == 2 && rounds <= 16;
  err = launch_product<CW, false>(P, P.nW, s, per_tile);
  if (err != hipSuccess) return err;
  if (a.mid_event && (err = hipEventRecord(a.mid_event, s)) != hipSuccess) return err;
  return launch_product<CX, true>(P, P.nX, s, per_tile);
}

// Tile choice: 256x256 dW tiles; 256-row dX tiles when experts keep many rows
// on average (MFMA-bound), 64-row dX tiles otherwise (a 256-row tile over an
// expert of a few dozen rows would spend most of its MFMAs on zero rows).
// LRM_GEMM_TILE=S|M|L|X overrides (benchmarking).
int gemm_tile_choice(const GemmArgs& a) {
  const char* env = getenv("LRM_GEMM_TILE");
  if (env && env[0] == 'S') return 0;
  if (env && env[0] == 'M') return 1;
  if (env && env[0] == 'L') return 2;
  if (env && env[0] == 'X') return 3;
  const int64_t per_expert = a.E > 0 ? (int64_t)a.max_rows / a.E : 0;
  return per_expert >= 192 ? 2 : 3;
}

int gemm_dw_tiles_per_expert(const GemmArgs& a) {
  if (!a.bf16 || !a.dW) return 0;
  auto per = [&](int bm, int bn) { return ((a.d_out + bm - 1) / bm) * ((a.d_in + bn - 1) / bn); };
  switch (gemm_tile_choice(a)) {
    case 3:
    case 2: return per(CfgL::BM, CfgL::BN);
    case 1: return per(CfgM::BM, CfgM::BN);
    default: return per(CfgS::BM, CfgS::BN);
  }
}

int gemm_dx_tile_rows(const GemmArgs& a) {
  if (!a.bf16) return FBM;
  switch (gemm_tile_choice(a)) {
    case 3: return CfgXS::BM;
    case 2: return CfgL::BM;
    case 1: return CfgM::BM;
    default: return CfgS::BM;
  }
}

hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t s) {
  if (!a.offsets || !a.mt_off || a.E < 1 || a.E > kPlanMaxE || (a.dXp && (!a.W || !a.Gp)) ||
      (a.dW && !a.Gp) ||
      (a.dW && a.max_rows > 0 && !a.Xp && !a.xrow) ||
      (a.Gp2 && (!a.W2 || a.d_out2 != a.d_out)))
    return hipErrorInvalidValue;
  if (a.xrow && (!a.bf16 || !a.xsrc || !a.xw || a.xsrc_rows * a.ldxs * 2 >= (1ll << 31) ||
                 a.ldxs < a.d_in))
    return hipErrorInvalidValue;
  // the row stride of Gp (Gp2) and the split dW: bf16 kernels only; a split
  // on a multiple of the waves' 64 rows
  if (a.lda != 0 && (!a.bf16 || a.lda < a.d_out || a.lda % 8)) return hipErrorInvalidValue;
  if (a.dw_split != 0 && (!a.bf16 || !a.dW || !a.dW2 || a.xrow || a.dw_split < 0 ||
                          a.dw_split >= a.d_out || a.dw_split % 64))
    return hipErrorInvalidValue;
  if (a.bf16) {
    // 32-bit store offsets inside a tile (the public entry points check this)
    if (a.d_in >= (1 << 20) || a.d_out >= (1 << 20)) return hipErrorInvalidValue;
    switch (gemm_tile_choice(a)) {
      case 3: return launch_bf16<CfgL, CfgXS>(a, s);
      case 2: return launch_bf16<CfgL, CfgL>(a, s);
      case 1: return launch_bf16<CfgM, CfgM>(a, s);
      default: return launch_bf16<CfgS, CfgS>(a, s);
    }
  }
  if (a.dw_bf16) return hipErrorInvalidValue;  // bf16 dW needs the bf16 kernels
  GemmPlan P{};
  hipError_t err = plan_tiles(a, FBM, FBN, FBM, FBN, &P, s);
  if (err != hipSuccess || P.G == 0) return err;
  LRM_LAUNCH(P.G, NT, 0, s, k_grouped_gemm_f32)(P);
  // one launch holds both tile kinds: the mid point is its end
  if (a.mid_event) {
    err = hipEventRecord(a.mid_event, s);
    if (err != hipSuccess) return err;
  }
  return hipGetLastError();
}

}  // namespace lrm

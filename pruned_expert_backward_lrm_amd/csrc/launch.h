// Internal launchers of the LRM kernels (host side).  Not part of the ABI.
#pragma once

#include <stdint.h>

#include "platform.h"

namespace lrm {

// Pairs per bucketing block: at least 256, and at most 1024 blocks.
inline int bucket_chunk(int N) {
  const int c = (N + 1023) / 1024;
  return c <= 256 ? 256 : (c + 63) / 64 * 64;
}
inline int bucket_blocks(int N) { return (N + bucket_chunk(N) - 1) / bucket_chunk(N); }

// --------------------------------------------------------------- score
hipError_t launch_row_sumsq(const void* M, int bf16, int64_t ld, int cols, int rows,
                            double* out, hipStream_t s);

struct ScoreOperands {
  int N, T, bf16;
  const int32_t* token;
  const float* weight;
  // g factor: PAIR rows reduced inline (gtab == nullptr) or a table indexed by
  // token (g_pair = 0) or by pair (g_pair = 1)
  const void* G; int64_t ldg; int gcols; const double* gtab; int g_pair;
  // x factor: same conventions; glu = 1 forms silu(A) * B rows inline instead
  const void* X; int64_t ldx; int xcols; const double* xtab; int x_pair;
  int glu; const void* A; const void* B; int64_t lda, ldb; int icols;
  float* score;
};
hipError_t launch_pair_score(const ScoreOperands& op, hipStream_t s);

// -------------------------------------------------------------- select
// Quotas of at most kQuotaPackMax experts, passed by value in the kernel
// arguments (2 KB): the host array is read at the call, and no copy
// operation is enqueued on the stream.
// (The CPU-emulation test build lowers it, so that its copy path runs on
// problems small enough to emulate.)
#ifndef LRM_QUOTA_PACK_MAX
#define LRM_QUOTA_PACK_MAX 512
#endif
constexpr int kQuotaPackMax = LRM_QUOTA_PACK_MAX;
struct QuotaPack {
  int32_t q[kQuotaPackMax];
};

struct BucketArgs {
  int N, T, E;
  const int32_t* token;
  const int32_t* expert;
  const int32_t* quota;  // device [E], or nullptr: qpack, or keep all
  const QuotaPack* qpack;  // host: quotas by value (E <= kQuotaPackMax), or nullptr
  const float* score;    // nullptr: no keys gathered
  int32_t* blkcnt;       // [E][bucket_blocks(N)]
  int32_t* cand_off;     // [E+1]
  int32_t* offsets;      // [E+1] kept offsets
  int32_t* cand;         // [N]
  uint32_t* keys;        // [N] or nullptr
  int32_t* pos;          // [N]
  int keep_all;          // pos written here (every valid pair kept, cand = kept)
  uint32_t* err;         // one word: the error bits of this call
  uint32_t* blkerr;      // [bucket_blocks(N)] per-block error bits (scratch)
  int32_t* tok_off;      // [T+1] first pair of each token, or nullptr (not wanted)
  int32_t* mt_off;       // [E+1] row-tile prefix of the kept blocks for dX tiles
  int mt_bm;             //   of mt_bm rows (mt_off == nullptr: not wanted)
  int64_t max_kept;      // rows the packed buffers hold (-1: no limit); more kept
                         //   rows set kErrCapacity
};
hipError_t launch_bucket(const BucketArgs& a, hipStream_t s);
// Per-block expert histograms of the pairs (the first bucketing step):
// blkcnt[e][b] pairs of expert e in block b of bucket_blocks(N), blkerr[b] the
// block's index-error bits; tok_off as in BucketArgs, or nullptr.
hipError_t launch_bucket_count(int N, int T, int E, const int32_t* token, const int32_t* expert,
                               int32_t* blkcnt, uint32_t* blkerr, int32_t* tok_off,
                               hipStream_t s);
// limit: candidate indices, packed slots and pos entries at or beyond it are
// never touched (the extent of keys, cand, pos and kept).
hipError_t launch_select(int E, const int32_t* cand_off, const int32_t* offsets,
                         const uint32_t* keys, const int32_t* cand, int32_t* pos, int32_t* kept,
                         int limit, hipStream_t s);
// quota: device [E]; or qpack (host, by value, E <= kQuotaPackMax) when quota
// is nullptr; both nullptr: keep all.  More than cap kept rows (cap >= 0) set
// kErrCapacity in err[0].
// The selection of a small call in one launch (the bucketing kernels and
// launch_select together), keep_all == 0 and keys gathered: same outputs.
// select_one_launch_ok(N, E) says whether it applies (LRM_SELECT_ONE_LAUNCH=0
// turns it off).
bool select_one_launch_ok(int N, int E);
hipError_t launch_select_one(const BucketArgs& b, int32_t* kept, int limit, hipStream_t s);
hipError_t launch_kept_offsets(int E, const int32_t* cand_off, const int32_t* quota,
                               const QuotaPack* qpack, int32_t* offsets, uint32_t* err,
                               int64_t cap, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t s);
hipError_t launch_token_offsets(int N, int T, const int32_t* token, int32_t* tok_off,
                                hipStream_t s);
hipError_t launch_tile_plan(int E, int bm, const int32_t* offsets, int32_t* mt_off,
                            hipStream_t s);

// --------------------------------------------------------- quota control
// Water-filling quotas on the device.  counts: device [E], or nullptr to
// count the pairs (token, expert of N pairs, T tokens) with the bucketing
// histogram (blkcnt [E][bucket_blocks(N)], blkerr [bucket_blocks(N)] scratch;
// the pairs' index errors go to err[0]).
struct QuotaArgs {
  int N, T, E;
  const int32_t* token;
  const int32_t* expert;
  const int32_t* counts;
  int64_t budget;
  int32_t* quota;
  int32_t* blkcnt;
  uint32_t* blkerr;
  uint32_t* err;
};
hipError_t launch_quota_waterfill(const QuotaArgs& a, hipStream_t s);

// ------------------------------------------------------------- compact
// Row j < min(offsets[E], max_rows) of the packed block:
//   a = kept[j]; p = pairmap ? pairmap[a] : a
//   Xp[j] = w_p * X[x_pair ? p : token[p]]            (glu = 0)
//   Xp[j] = w_p * silu(X[p]) * X2[p]                  (glu = 1, PAIR rows)
//   Gp[j] = G[g_by_id ? a : (g_pair ? p : token[p])]
// written to row dst[j] instead of j when dst is given (rows outside
// [0, max_rows) are skipped).
struct CompactArgs {
  int T, bf16, max_rows, E;
  const int32_t* offsets;
  const int32_t* kept;
  const int32_t* dst;
  const int32_t* pairmap;
  const int32_t* token;
  const float* weight;
  const void* X; int64_t ldx; int xcols; int x_pair; void* Xp;
  int glu; const void* X2; int64_t ldx2;
  const void* G; int64_t ldg; int gcols; int g_pair; int g_by_id; void* Gp;
};
hipError_t launch_compact(const CompactArgs& a, hipStream_t s);
// The row map of the gathering GEMM loader instead of a packed copy: for
// packed row j < min(offsets[E], max_rows), p = kept[j]:
//   xrow[j] = x_pair ? p : token[p];  xw[j] = weight[p]
hipError_t launch_row_map(const CompactArgs& a, int32_t* xrow, float* xw, hipStream_t s);

// --------------------------------------------------------- grouped GEMM
// For each expert e with packed rows [offsets[e], offsets[e+1]):
//   dW[e]  = Gp_e^T Xp_e                 [d_out][d_in]
//   dXp_e  = Gp_e W_e (+ Gp2_e W2_e)     [M_e][d_in]   (second term optional)
struct GemmArgs {
  int E, bf16, max_rows, d_in, d_out;
  const int32_t* offsets;
  const void* Gp;  // [rows][d_out], rows lda apart (bf16 kernels; lda 0: d_out)
  int lda;
  const void* Xp;  // [rows][d_in]
  const void* W; int64_t w_stride;  // [E][d_out][d_in]
  const void* Gp2; const void* W2; int64_t w2_stride; int d_out2;  // optional
  // dW split in two outputs (bf16 kernels; dw_split 0: one output): rows
  // [0, dw_split) of each expert's dW go to dW ([E][dw_split][d_in]) and rows
  // [dw_split, d_out) to dW2 ([E][d_out - dw_split][d_in]); dw_split is a
  // multiple of 64, so every wave of a tile writes to one of them
  float* dW2;
  int dw_split;
  float* dW;   // [E][d_out][d_in] or nullptr
  float* dXp;  // [max_rows][d_in] or nullptr
  int32_t* mt_off;  // workspace [gemm_workspace_ints(E)]: the dX row-tile prefix [E+1], then the dW schedule
  int mt_ready;     // mt_off already holds the prefix for gemm_dx_tile_rows(*this)
  int dw_bf16;      // dW is stored as bf16 (round to nearest even), bf16 kernels only
  hipEvent_t mid_event;  // recorded after the dW launch, before the dX launch (or null)
  // dW with the B operand gathered by its loader instead of read from Xp
  // (bf16 only; xrow != nullptr): packed row m of B is
  // bf16(xw[m] * xsrc[xrow[m]]), the value compaction would have written;
  // xsrc has xsrc_rows rows of leading dimension ldxs, under 2 GiB.
  const void* xsrc; int64_t ldxs; int64_t xsrc_rows;
  const int32_t* xrow; const float* xw;
  int32_t* dw_plan;  // set by launch_grouped_gemm (inside the mt_off workspace)
  // the workspace already holds the dW schedule of a launch with the same
  // offsets, max_rows and gemm_dw_tiles_per_expert (the schedule depends on
  // nothing else)
  int dw_plan_ready;
  // host pointer, or null: when this launch plans its dW schedule, the same
  // plan launch also writes the schedule of *dw_plan_next (a later bf16 dW
  // launch with the same E, offsets and max_rows, into its own mt_off
  // workspace), which then runs with dw_plan_ready
  const GemmArgs* dw_plan_next;
};
// int32 entries of the grouped GEMM's workspace for E experts
int64_t gemm_workspace_ints(int E);
// dW tiles per expert of the bf16 kernels (0: no scheduled dW launch)
int gemm_dw_tiles_per_expert(const GemmArgs& a);
int gemm_tile_choice(const GemmArgs& a);
// Rows of a dX tile of the bf16 kernels (the prefix mt_off is built for it).
int gemm_dx_tile_rows(const GemmArgs& a);
hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t s);

// ------------------------------------------------------------ unpermute
// Up to two sources; the row of pair p in source k is
//   r = pos_k[p]; if (r >= 0 && pos2_k) r = pos2_k[r];
// with r taken as missing when it reaches past pos2_rows[k] (before the
// second lookup) or src_rows[k] (the rows source k holds).
struct ScatterArgs {
  int N, T, d, out_pair;
  const int32_t* token;
  const float* weight;
  const int32_t* tok_off;  // [T+1] (TOKEN output)
  const int32_t* pos[2];
  const int32_t* pos2[2];
  const float* src[2];
  int pos2_rows[2];
  int src_rows[2];
  float* dX;
};
hipError_t launch_unpermute(const ScatterArgs& a, hipStream_t s);

// --------------------------------------------------------- SwiGLU backward
// For down-kept row m < min(offsets_down[E], max_rows), p = kept_down[m]:
//   u = U[m]; a = A[p]; b = B[p]
//   ga = u * b * silu'(a) -> GA[m];  gb = u * silu(a) -> GB[m]
//   s_gate[m] = w^2 |ga|^2 x2[row of p];  s_up[m] = w^2 |gb|^2 x2[row of p]
struct GluBwdArgs {
  int T, bf16, max_rows, E, I;
  const int32_t* offsets_down;
  const int32_t* kept_down;
  const int32_t* token;
  const float* weight;
  const float* U;  // [rows][I] fp32
  const void* A; int64_t lda;
  const void* B; int64_t ldb;
  const double* x2; int x_pair;
  void* GA; void* GB;  // [rows][I], rows ldg apart (0: I)
  int ldg;
  float* s_gate; float* s_up;
};
hipError_t launch_glu_bwd(const GluBwdArgs& a, hipStream_t s);

}  // namespace lrm

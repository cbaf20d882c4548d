// Host side of the C ABI declared in include/lrm.h: argument validation,
// workspace planning and the stream-ordered launch sequences.  Nothing here
// allocates device memory; scratch comes from the caller's workspace.
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include "lrm.h"
#include "common.h"
#include "launch.h"

using namespace lrm;

namespace {

constexpr int kMaxE = 4096;
// GEMM leading dimensions: a 256-row output tile spans less than 1 GiB, so
// its stores take 32-bit offsets
constexpr int kMaxDim = (1 << 20) - 1;
constexpr size_t kAlign = 256;

// Bump allocator over a caller workspace.  With base == nullptr it only
// measures, so size queries and real calls carve identical layouts.
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(int64_t n) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += (size_t)(n > 0 ? n : 0) * sizeof(T);
    return p;
  }
  size_t size() const { return (off + kAlign - 1) / kAlign * kAlign; }
};

int esize(int dtype) { return dtype == LRM_BF16 ? 2 : 4; }

lrm_status check_pairs(const lrm_pairs* p) {
  if (!p) return LRM_ERR_NULL;
  if (p->T < 0 || p->N < 0 || p->E < 1 || p->E > kMaxE) return LRM_ERR_SHAPE;
  if (p->N > 0 && (!p->token || !p->expert || !p->weight)) return LRM_ERR_NULL;
  return LRM_OK;
}

// A dense input: dtype, layout, shape, 16-byte row alignment.
lrm_status check_mat(const lrm_mat* m, const lrm_pairs* p, int dtype, int cols, int need_rows) {
  if (!m) return LRM_ERR_NULL;
  if (m->dtype != LRM_F32 && m->dtype != LRM_BF16) return LRM_ERR_DTYPE;
  if (m->dtype != dtype) return LRM_ERR_DTYPE;
  if (m->rows != LRM_ROWS_TOKEN && m->rows != LRM_ROWS_PAIR) return LRM_ERR_LAYOUT;
  if (need_rows >= 0 && m->rows != need_rows) return LRM_ERR_LAYOUT;
  if (m->cols <= 0 || (cols >= 0 && m->cols != cols)) return LRM_ERR_SHAPE;
  if (m->ld < m->cols) return LRM_ERR_SHAPE;
  if (m->cols % (16 / esize(m->dtype)) != 0) return LRM_ERR_UNSUPPORTED;
  const int64_t nrows = m->rows == LRM_ROWS_TOKEN ? p->T : p->N;
  if (nrows > 0 && !m->ptr) return LRM_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(m->ptr) & 15u) != 0) return LRM_ERR_ALIGN;
  if ((m->ld * esize(m->dtype)) % 16 != 0) return LRM_ERR_ALIGN;
  return LRM_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

lrm_status check_quota(const int32_t* q, int E, int64_t* sum) {
  if (!q) return LRM_ERR_NULL;
  int64_t s = 0;
  for (int e = 0; e < E; ++e) {
    if (q[e] < 0) return LRM_ERR_QUOTA;
    s += q[e];
  }
  if (sum) *sum = s;
  return LRM_OK;
}

#define LRM_TRY_HIP(x)                        \
  do {                                        \
    if ((x) != hipSuccess) return LRM_ERR_HIP; \
  } while (0)
#define LRM_TRY(x)                  \
  do {                              \
    lrm_status st_ = (x);           \
    if (st_ != LRM_OK) return st_;  \
  } while (0)

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Host quotas of more than kQuotaPackMax experts are copied into the
// workspace with a stream copy of the host array.  A captured graph would
// re-read that array at every replay while keeping the packed sizes the host
// computed from it at capture, so such a call is refused under capture
// (device quotas, or at most kQuotaPackMax experts, are the capturable forms).
lrm_status check_capturable(int E, bool host_quotas, hipStream_t s) {
  if (!host_quotas || E <= kQuotaPackMax) return LRM_OK;
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess) return LRM_ERR_HIP;
  return st == hipStreamCaptureStatusNone ? LRM_OK : LRM_ERR_UNSUPPORTED;
}

// ---------------------------------------------------------------- scoring

struct ScoreWs {
  double* gtab;
  double* xtab;
};

ScoreWs carve_score(Carve& c, int T) {
  ScoreWs w;
  w.gtab = c.take<double>(T);
  w.xtab = c.take<double>(T);
  return w;
}

// Launch the norm tables of TOKEN-layout operands and the pair kernel.
hipError_t run_score(const lrm_pairs* p, const lrm_mat* X, const lrm_mat* G, float* score,
                     const ScoreWs& w, hipStream_t s) {
  const int bf16 = X->dtype == LRM_BF16;
  ScoreOperands op{};
  op.N = p->N; op.T = p->T; op.bf16 = bf16; op.token = p->token; op.weight = p->weight;
  op.G = G->ptr; op.ldg = G->ld; op.gcols = G->cols; op.g_pair = G->rows == LRM_ROWS_PAIR;
  op.X = X->ptr; op.ldx = X->ld; op.xcols = X->cols; op.x_pair = X->rows == LRM_ROWS_PAIR;
  op.score = score;
  if (!op.g_pair) {
    hipError_t e = launch_row_sumsq(G->ptr, bf16, G->ld, G->cols, p->T, w.gtab, s);
    if (e != hipSuccess) return e;
    op.gtab = w.gtab;
  }
  if (!op.x_pair) {
    hipError_t e = launch_row_sumsq(X->ptr, bf16, X->ld, X->cols, p->T, w.xtab, s);
    if (e != hipSuccess) return e;
    op.xtab = w.xtab;
  }
  return launch_pair_score(op, s);
}

// h_tab (optional): |silu(a) * b|^2 of every pair, saved by the forward; the
// pair kernel then reads it instead of the A and B rows.
hipError_t run_score_glu(const lrm_pairs* p, const lrm_mat* A, const lrm_mat* B,
                         const lrm_mat* G, float* score, const ScoreWs& w, hipStream_t s,
                         const double* h_tab = nullptr) {
  const int bf16 = A->dtype == LRM_BF16;
  ScoreOperands op{};
  op.N = p->N; op.T = p->T; op.bf16 = bf16; op.token = p->token; op.weight = p->weight;
  op.G = G->ptr; op.ldg = G->ld; op.gcols = G->cols; op.g_pair = G->rows == LRM_ROWS_PAIR;
  if (h_tab) {
    op.xtab = h_tab;
  } else {
    op.glu = 1; op.A = A->ptr; op.B = B->ptr; op.lda = A->ld; op.ldb = B->ld;
    op.icols = A->cols;
  }
  op.x_pair = 1;
  op.score = score;
  if (!op.g_pair) {
    hipError_t e = launch_row_sumsq(G->ptr, bf16, G->ld, G->cols, p->T, w.gtab, s);
    if (e != hipSuccess) return e;
    op.gtab = w.gtab;
  }
  return launch_pair_score(op, s);
}

// ---------------------------------------------------------------- selection

struct SelectWs {
  uint32_t* err;
  uint32_t* blkerr;
  int32_t* quota;
  int32_t* blkcnt;
  int32_t* cand_off;
  int32_t* cand;
  uint32_t* keys;
};

SelectWs carve_select(Carve& c, int N, int E) {
  SelectWs w;
  w.err = c.take<uint32_t>(64);
  w.blkerr = c.take<uint32_t>(bucket_blocks(N));
  w.quota = c.take<int32_t>(E);
  w.blkcnt = c.take<int32_t>((int64_t)bucket_blocks(N) * E);
  w.cand_off = c.take<int32_t>(E + 1);
  w.cand = c.take<int32_t>(N);
  w.keys = c.take<uint32_t>(N);
  return w;
}

// Bucket the pairs by expert and select the top quota of each expert.
// quota_host == nullptr keeps everything (then kept is filled by the bucket
// scatter and no keys are gathered); with quota_on_device it is a device
// pointer, used as it is.
// tok_off (optional, [T+1]): the first pair of each token, computed on the way
// when there is at least one pair.  mt_off (optional, [E+1]): the prefix of
// ceil(M_e / mt_bm), the dX row tiles of the grouped GEMM.  max_kept: the rows
// the packed buffers were sized for (-1: none); more kept rows are flagged in
// the error word.
lrm_status run_select(const lrm_pairs* p, const float* score, const int32_t* quota_host,
                      int32_t* pos, int32_t* offsets, int32_t* kept, const SelectWs& w,
                      hipStream_t s, int32_t* tok_off = nullptr, int32_t* mt_off = nullptr,
                      int mt_bm = 0, bool quota_on_device = false, int64_t max_kept = -1) {
  const bool keep_all = quota_host == nullptr;
  // host quotas of up to kQuotaPackMax experts go by value with the scan's
  // launch; more are copied stream-ordered into the workspace
  const bool by_value = !keep_all && !quota_on_device && p->E <= kQuotaPackMax;
  QuotaPack pack;
  if (by_value) std::memcpy(pack.q, quota_host, sizeof(int32_t) * p->E);
  if (!keep_all && !quota_on_device && !by_value) {
    LRM_TRY_HIP(hipMemcpyAsync(w.quota, quota_host, sizeof(int32_t) * p->E,
                               hipMemcpyHostToDevice, s));
  }
  BucketArgs b{};
  b.N = p->N; b.T = p->T; b.E = p->E; b.token = p->token; b.expert = p->expert;
  b.quota = keep_all || by_value ? nullptr : (quota_on_device ? quota_host : w.quota);
  b.qpack = by_value ? &pack : nullptr;
  b.score = keep_all ? nullptr : score;
  b.blkcnt = w.blkcnt; b.cand_off = w.cand_off; b.offsets = offsets;
  b.cand = keep_all ? kept : w.cand;
  b.keys = keep_all ? nullptr : w.keys;
  b.pos = pos; b.keep_all = keep_all; b.err = w.err; b.blkerr = w.blkerr; b.tok_off = tok_off;
  b.mt_off = mt_off; b.mt_bm = mt_bm; b.max_kept = max_kept;
  if (!keep_all && select_one_launch_ok(p->N, p->E)) {
    LRM_TRY_HIP(launch_select_one(b, kept, p->N, s));
    return LRM_OK;
  }
  LRM_TRY_HIP(launch_bucket(b, s));
  if (!keep_all)
    LRM_TRY_HIP(launch_select(p->E, w.cand_off, offsets, w.keys, w.cand, pos, kept, p->N, s));
  return LRM_OK;
}

}  // namespace

// =========================================================== the C ABI

extern "C" {

const char* lrm_status_string(lrm_status s) {
  switch (s) {
    case LRM_OK: return "ok";
    case LRM_ERR_NULL: return "a required pointer is NULL";
    case LRM_ERR_SHAPE: return "inconsistent or unsupported sizes";
    case LRM_ERR_DTYPE: return "unknown or mixed dtype";
    case LRM_ERR_LAYOUT: return "unknown or unsupported row layout";
    case LRM_ERR_ALIGN: return "rows are not 16-byte aligned";
    case LRM_ERR_QUOTA: return "negative quota";
    case LRM_ERR_WORKSPACE: return "workspace missing or too small";
    case LRM_ERR_INDEX: return "expert or token index out of range or out of order, or an assignment not matching the kept counts";
    case LRM_ERR_HIP: return "HIP runtime error";
    case LRM_ERR_UNSUPPORTED: return "unsupported request";
    case LRM_ERR_INFEASIBLE: return "kept pairs that no replica or capacity can take";
  }
  return "unknown status";
}

int32_t lrm_version(void) { return 100; }

int64_t lrm_max_kept(int32_t N, int32_t E, const int32_t* quota) {
  if (!quota || E < 1) return -1;
  int64_t s = 0;
  if (check_quota(quota, E, &s) != LRM_OK) return -1;
  return s < N ? s : N;
}

size_t lrm_score_workspace_size(const lrm_pairs* pairs) {
  if (check_pairs(pairs) != LRM_OK) return 0;
  Carve c(nullptr);
  carve_score(c, pairs->T);
  return c.size();
}

lrm_status lrm_score(const lrm_pairs* pairs, const lrm_mat* X, const lrm_mat* G, float* score,
                     void* ws, size_t ws_bytes, void* stream) {
  LRM_TRY(check_pairs(pairs));
  if (!X || !G) return LRM_ERR_NULL;
  LRM_TRY(check_mat(X, pairs, X->dtype, -1, -1));
  LRM_TRY(check_mat(G, pairs, X->dtype, -1, -1));
  if (pairs->N > 0 && !score) return LRM_ERR_NULL;
  Carve c(nullptr);
  carve_score(c, pairs->T);
  if (!ws || ws_bytes < c.size()) return LRM_ERR_WORKSPACE;
  Carve r(ws);
  ScoreWs w = carve_score(r, pairs->T);
  LRM_TRY_HIP(run_score(pairs, X, G, score, w, as_stream(stream)));
  return LRM_OK;
}

lrm_status lrm_score_glu(const lrm_pairs* pairs, const lrm_mat* A, const lrm_mat* B,
                         const lrm_mat* G, float* score, void* ws, size_t ws_bytes,
                         void* stream) {
  LRM_TRY(check_pairs(pairs));
  if (!A || !B || !G) return LRM_ERR_NULL;
  LRM_TRY(check_mat(A, pairs, A->dtype, -1, LRM_ROWS_PAIR));
  LRM_TRY(check_mat(B, pairs, A->dtype, A->cols, LRM_ROWS_PAIR));
  LRM_TRY(check_mat(G, pairs, A->dtype, -1, -1));
  if (pairs->N > 0 && !score) return LRM_ERR_NULL;
  Carve c(nullptr);
  carve_score(c, pairs->T);
  if (!ws || ws_bytes < c.size()) return LRM_ERR_WORKSPACE;
  Carve r(ws);
  ScoreWs w = carve_score(r, pairs->T);
  LRM_TRY_HIP(run_score_glu(pairs, A, B, G, score, w, as_stream(stream)));
  return LRM_OK;
}

size_t lrm_select_workspace_size(const lrm_pairs* pairs) {
  if (check_pairs(pairs) != LRM_OK) return 0;
  Carve c(nullptr);
  carve_select(c, pairs->N, pairs->E);
  return c.size();
}

lrm_status lrm_select(const lrm_pairs* pairs, const float* score, const int32_t* quota,
                      uint32_t flags, int32_t* pos, int32_t* offsets, int32_t* kept, void* ws,
                      size_t ws_bytes, void* stream) {
  LRM_TRY(check_pairs(pairs));
  const bool keep_all = (flags & LRM_KEEP_ALL) != 0;
  const bool qdev = (flags & LRM_QUOTA_ON_DEVICE) != 0;
  if (flags & ~(LRM_KEEP_ALL | LRM_QUOTA_ON_DEVICE)) return LRM_ERR_UNSUPPORTED;
  if (!offsets) return LRM_ERR_NULL;
  if (pairs->N > 0 && (!pos || !kept)) return LRM_ERR_NULL;
  if (!keep_all) {
    if (pairs->N > 0 && !score) return LRM_ERR_NULL;
    if (qdev) {
      if (!quota) return LRM_ERR_NULL;
    } else {
      LRM_TRY(check_quota(quota, pairs->E, nullptr));
    }
  }
  Carve c(nullptr);
  carve_select(c, pairs->N, pairs->E);
  if (!ws || ws_bytes < c.size()) return LRM_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  LRM_TRY(check_capturable(pairs->E, !keep_all && !qdev, s));
  Carve r(ws);
  SelectWs w = carve_select(r, pairs->N, pairs->E);
  return run_select(pairs, score, keep_all ? nullptr : quota, pos, offsets, kept, w, s, nullptr,
                    nullptr, 0, qdev);
}

}  // extern "C"

// Scratch of lrm_select_static: one array per GPU, loaded with the code
// object and held until the process ends.  Host code never uses its name as
// an address: the device address comes from hipGetSymbolAddress, taken once
// per device with that device current.
static __device__ __align__(256) unsigned char scratch[LRM_SELECT_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's copy of scratch.
lrm_status static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LRM_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return LRM_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LRM_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LRM_OK;
}

}  // namespace

extern "C" {

lrm_status lrm_select_static(const lrm_pairs* pairs, const float* score, const int32_t* quota,
                             uint32_t flags, int32_t* pos, int32_t* offsets, int32_t* kept,
                             void* stream) {
  LRM_TRY(check_pairs(pairs));
  if (lrm_select_workspace_size(pairs) > (size_t)LRM_SELECT_STATIC_SCRATCH_BYTES)
    return LRM_ERR_WORKSPACE;
  void* ws = nullptr;
  LRM_TRY(static_scratch(&ws));
  // every scratch word the selection reads is written earlier in the same
  // call, so the previous call's contents need no clearing
  return lrm_select(pairs, score, quota, flags, pos, offsets, kept, ws,
                    LRM_SELECT_STATIC_SCRATCH_BYTES, stream);
}

lrm_status lrm_compact(const lrm_pairs* pairs, const int32_t* kept, const int32_t* offsets,
                       int32_t max_rows, const lrm_mat* X, const lrm_mat* G, void* Xp, void* Gp,
                       void* stream) {
  return lrm_compact_rows(pairs, kept, offsets, max_rows, nullptr, X, G, Xp, Gp, stream);
}

lrm_status lrm_compact_rows(const lrm_pairs* pairs, const int32_t* kept, const int32_t* offsets,
                            int32_t max_rows, const int32_t* dst, const lrm_mat* X,
                            const lrm_mat* G, void* Xp, void* Gp, void* stream) {
  LRM_TRY(check_pairs(pairs));
  if (!X || !G) return LRM_ERR_NULL;
  LRM_TRY(check_mat(X, pairs, X->dtype, -1, -1));
  LRM_TRY(check_mat(G, pairs, X->dtype, -1, -1));
  if (max_rows < 0) return LRM_ERR_SHAPE;
  if (!offsets || (max_rows > 0 && !kept)) return LRM_ERR_NULL;
  if ((Xp && !aligned16(Xp)) || (Gp && !aligned16(Gp))) return LRM_ERR_ALIGN;
  CompactArgs a{};
  a.T = pairs->T; a.bf16 = X->dtype == LRM_BF16; a.max_rows = max_rows; a.E = pairs->E;
  a.offsets = offsets; a.kept = kept; a.dst = dst; a.token = pairs->token;
  a.weight = pairs->weight;
  a.X = X->ptr; a.ldx = X->ld; a.xcols = X->cols; a.x_pair = X->rows == LRM_ROWS_PAIR; a.Xp = Xp;
  a.G = G->ptr; a.ldg = G->ld; a.gcols = G->cols; a.g_pair = G->rows == LRM_ROWS_PAIR; a.Gp = Gp;
  LRM_TRY_HIP(launch_compact(a, as_stream(stream)));
  return LRM_OK;
}

size_t lrm_grouped_bwd_workspace_size(int32_t E) {
  if (E < 1 || E > kMaxE) return 0;
  Carve c(nullptr);
  c.take<int32_t>(gemm_workspace_ints(E));
  return c.size();
}

lrm_status lrm_grouped_bwd(int32_t E, const int32_t* offsets, int32_t max_rows, int32_t dtype,
                           const void* Gp, const void* Xp, const void* W, int64_t w_stride,
                           int32_t d_in, int32_t d_out, float* dW, float* dXp, void* ws,
                           size_t ws_bytes, void* stream) {
  if (E < 1 || E > kMaxE || max_rows < 0 || d_in <= 0 || d_out <= 0 || d_in > kMaxDim ||
      d_out > kMaxDim)
    return LRM_ERR_SHAPE;
  if (dtype != LRM_F32 && dtype != LRM_BF16) return LRM_ERR_DTYPE;
  const int q = 16 / esize(dtype);
  if (d_in % q || d_out % q) return LRM_ERR_UNSUPPORTED;
  if (!offsets) return LRM_ERR_NULL;
  if (max_rows > 0 && !Gp) return LRM_ERR_NULL;
  if (dW && max_rows > 0 && !Xp) return LRM_ERR_NULL;
  if (dXp && !W) return LRM_ERR_NULL;
  if (dXp && w_stride < (int64_t)d_in * d_out) return LRM_ERR_SHAPE;
  if (!aligned16(Gp) || !aligned16(Xp) || !aligned16(W) || !aligned16(dW) || !aligned16(dXp))
    return LRM_ERR_ALIGN;
  if (W && (w_stride * esize(dtype)) % 16) return LRM_ERR_ALIGN;
  if (!ws || ws_bytes < lrm_grouped_bwd_workspace_size(E)) return LRM_ERR_WORKSPACE;
  GemmArgs g{};
  g.E = E; g.bf16 = dtype == LRM_BF16; g.max_rows = max_rows; g.d_in = d_in; g.d_out = d_out;
  g.offsets = offsets; g.Gp = Gp; g.Xp = Xp; g.W = W; g.w_stride = w_stride;
  g.dW = dW; g.dXp = dXp;
  Carve r(ws);
  g.mt_off = r.take<int32_t>(gemm_workspace_ints(E));
  LRM_TRY_HIP(launch_grouped_gemm(g, as_stream(stream)));
  return LRM_OK;
}

size_t lrm_unpermute_workspace_size(const lrm_pairs* pairs) {
  if (check_pairs(pairs) != LRM_OK) return 0;
  Carve c(nullptr);
  c.take<int32_t>((int64_t)pairs->T + 1);
  return c.size();
}

lrm_status lrm_unpermute(const lrm_pairs* pairs, const int32_t* pos, const float* dXp,
                         int32_t d_in, int32_t out_rows, float* dX, void* ws, size_t ws_bytes,
                         void* stream) {
  LRM_TRY(check_pairs(pairs));
  if (out_rows != LRM_ROWS_TOKEN && out_rows != LRM_ROWS_PAIR) return LRM_ERR_LAYOUT;
  if (d_in <= 0) return LRM_ERR_SHAPE;
  if (d_in % 4) return LRM_ERR_UNSUPPORTED;
  const int64_t rows = out_rows == LRM_ROWS_TOKEN ? pairs->T : pairs->N;
  if (rows > 0 && !dX) return LRM_ERR_NULL;
  if (pairs->N > 0 && (!pos || !dXp)) return LRM_ERR_NULL;
  if (!aligned16(dX) || !aligned16(dXp)) return LRM_ERR_ALIGN;
  if (!ws || ws_bytes < lrm_unpermute_workspace_size(pairs)) return LRM_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  ScatterArgs a{};
  a.N = pairs->N; a.T = pairs->T; a.d = d_in; a.out_pair = out_rows == LRM_ROWS_PAIR;
  a.token = pairs->token; a.weight = pairs->weight;
  a.pos[0] = pos; a.src[0] = dXp;
  a.src_rows[0] = 0x7fffffff;  // the caller's dXp holds every row pos names
  a.dX = dX;
  if (!a.out_pair) {
    Carve r(ws);
    int32_t* tok_off = r.take<int32_t>((int64_t)pairs->T + 1);
    LRM_TRY_HIP(launch_token_offsets(pairs->N, pairs->T, pairs->token, tok_off, s));
    a.tok_off = tok_off;
  }
  LRM_TRY_HIP(launch_unpermute(a, s));
  return LRM_OK;
}

size_t lrm_quota_waterfill_device_workspace_size(const lrm_pairs* pairs) {
  if (check_pairs(pairs) != LRM_OK) return 0;
  Carve c(nullptr);
  carve_select(c, pairs->N, pairs->E);
  return c.size();
}

lrm_status lrm_quota_waterfill_device(const lrm_pairs* pairs, const int32_t* counts,
                                      int64_t budget, int32_t* quota, void* ws, size_t ws_bytes,
                                      void* stream) {
  LRM_TRY(check_pairs(pairs));
  if (!quota) return LRM_ERR_NULL;
  if (budget < 0) return LRM_ERR_QUOTA;
  Carve c(nullptr);
  carve_select(c, pairs->N, pairs->E);
  if (!ws || ws_bytes < c.size()) return LRM_ERR_WORKSPACE;
  // the selection's layout: error word first, the histogram scratch as the
  // bucketing pass uses it
  Carve r(ws);
  SelectWs w = carve_select(r, pairs->N, pairs->E);
  QuotaArgs a{};
  a.N = pairs->N; a.T = pairs->T; a.E = pairs->E; a.token = pairs->token;
  a.expert = pairs->expert; a.counts = counts; a.budget = budget; a.quota = quota;
  a.blkcnt = w.blkcnt; a.blkerr = w.blkerr; a.err = w.err;
  LRM_TRY_HIP(launch_quota_waterfill(a, as_stream(stream)));
  return LRM_OK;
}

lrm_status lrm_check_device_errors(void* ws, void* stream) {
  if (!ws) return LRM_ERR_NULL;
  hipStream_t s = as_stream(stream);
  LRM_TRY_HIP(hipStreamSynchronize(s));
  uint32_t word = 0;
  LRM_TRY_HIP(hipMemcpy(&word, ws, sizeof(word), hipMemcpyDeviceToHost));
  if (word) {
    LRM_TRY_HIP(launch_fill_u32(static_cast<uint32_t*>(ws), 0u, 1, s));
    LRM_TRY_HIP(hipStreamSynchronize(s));
    // index errors first; capacity alone: the packed buffers were too small
    return (word & ~kErrCapacity) ? LRM_ERR_INDEX : LRM_ERR_WORKSPACE;
  }
  return LRM_OK;
}

}  // extern "C"

// ===================================================== the fused backward

namespace {

struct LinearPlan {
  int64_t Mcap;
  SelectWs sel;
  ScoreWs sc;
  float* score;
  int32_t* pos;
  int32_t* offsets;
  int32_t* kept;
  int32_t* tok_off;
  int32_t* mt_off;
  void* Gp;
  void* Xp;
  int32_t* xrow;  // gathering loaders: source row and weight of each packed row
  float* xw;
  float* dXp;
};

// LRM_GATHER_LOADS: the weight-gradient GEMM gathers its w*x operand from X
// (bf16, X under 2 GiB for the loader's 32-bit offsets) instead of reading a
// packed copy.
bool gather_loads(const lrm_problem* pb) {
  if (!(pb->flags & LRM_GATHER_LOADS) || pb->dtype != LRM_BF16) return false;
  const int64_t rows = pb->X.rows == LRM_ROWS_PAIR ? pb->pairs.N : pb->pairs.T;
  return rows * pb->X.ld * 2 < (1ll << 31);
}

LinearPlan carve_linear(Carve& c, const lrm_problem* pb, const lrm_outputs* out, int64_t Mcap) {
  const lrm_pairs& p = pb->pairs;
  const int es = esize(pb->dtype);
  LinearPlan L{};
  L.Mcap = Mcap;
  L.sel = carve_select(c, p.N, p.E);
  L.sc = carve_score(c, p.T);
  L.score = c.take<float>(p.N);
  L.pos = c.take<int32_t>(p.N);
  L.offsets = c.take<int32_t>(p.E + 1);
  L.kept = c.take<int32_t>(p.N);
  L.tok_off = c.take<int32_t>((int64_t)p.T + 1);
  L.mt_off = c.take<int32_t>(gemm_workspace_ints(p.E));
  L.Gp = c.take<char>(Mcap * pb->d_out * es);
  if (gather_loads(pb)) {
    L.xrow = c.take<int32_t>(Mcap);
    L.xw = c.take<float>(Mcap);
  } else {
    L.Xp = c.take<char>(Mcap * pb->d_in * es);
  }
  L.dXp = c.take<float>(Mcap * pb->d_in);
  if (out) {
    if (out->score) L.score = out->score;
    if (out->pos) L.pos = out->pos;
    if (out->offsets) L.offsets = out->offsets;
  }
  return L;
}

struct GluPlan {
  int64_t Md, Mg, Mu;
  bool pass_through;
  SelectWs sel;
  ScoreWs sc;
  double* x2;
  int32_t* qgate;
  int32_t* qup;
  float* score;
  int32_t* pos;
  int32_t* offsets;
  int32_t* kept;
  int32_t* tok_off;
  int32_t* mt_off;
  int32_t* mt_off2;  // the one gate/up dW launch's schedule (planned with the down one)
  void* Gd;      // [Md][H] g rows
  void* Hd;      // [Md][I] w * h rows
  float* U;      // [Md][I]
  void* GA;      // [Md][I]
  void* GB;      // [Md][I]
  float* s_gate; // [Md]
  float* s_up;   // [Md]
  int32_t* pos_g; int32_t* off_g; int32_t* kept_g;
  int32_t* pos_u; int32_t* off_u; int32_t* kept_u;
  void* Xgu;     // pass-through: [Md][H] w * x rows
  float* dXp;    // pass-through: [Md][H]
  void* GAp; void* Xg; float* dXg;  // separate: gate [Mg]
  void* GBp; void* Xu; float* dXu;  // separate: up [Mu]
  // gathering loaders: row maps of the x rows (pass-through: [Md]; separate:
  // gate [Mg], up [Mu])
  int32_t* xrow_g; float* xw_g;
  int32_t* xrow_u; float* xw_u;
};

GluPlan carve_glu(Carve& c, const lrm_problem* pb, const lrm_outputs* out, int64_t Md,
                  int64_t Mg, int64_t Mu, bool pass_through) {
  const lrm_pairs& p = pb->pairs;
  const int es = esize(pb->dtype);
  const int64_t H = pb->H, I = pb->I;
  GluPlan L{};
  L.Md = Md; L.Mg = Mg; L.Mu = Mu; L.pass_through = pass_through;
  L.sel = carve_select(c, p.N, p.E);
  L.sc = carve_score(c, p.T);
  L.x2 = c.take<double>(pb->X.rows == LRM_ROWS_PAIR ? p.N : p.T);
  L.qgate = c.take<int32_t>(p.E);
  L.qup = c.take<int32_t>(p.E);
  L.score = c.take<float>(p.N);
  L.pos = c.take<int32_t>(p.N);
  L.offsets = c.take<int32_t>(p.E + 1);
  L.kept = c.take<int32_t>(p.N);
  L.tok_off = c.take<int32_t>((int64_t)p.T + 1);
  L.mt_off = c.take<int32_t>(gemm_workspace_ints(p.E));
  L.mt_off2 = c.take<int32_t>(gemm_workspace_ints(p.E));
  L.Gd = c.take<char>(Md * H * es);
  L.Hd = c.take<char>(Md * I * es);
  L.U = c.take<float>(Md * I);
  // GA then GB, back to back: the fused gate/up path writes rows of [GA | GB]
  // (2I wide) into the span of both
  L.GA = c.take<char>(Md * I * es);
  L.GB = c.take<char>(Md * I * es);
  L.s_gate = c.take<float>(Md);
  L.s_up = c.take<float>(Md);
  L.pos_g = c.take<int32_t>(Md);
  L.off_g = c.take<int32_t>(p.E + 1);
  L.kept_g = c.take<int32_t>(Md);
  L.pos_u = c.take<int32_t>(Md);
  L.off_u = c.take<int32_t>(p.E + 1);
  L.kept_u = c.take<int32_t>(Md);
  const bool gl = gather_loads(pb);
  if (pass_through) {
    if (gl) {
      L.xrow_g = L.xrow_u = c.take<int32_t>(Md);
      L.xw_g = L.xw_u = c.take<float>(Md);
    } else {
      L.Xgu = c.take<char>(Md * H * es);
    }
    L.dXp = c.take<float>(Md * H);
  } else {
    L.GAp = c.take<char>(Mg * I * es);
    L.dXg = c.take<float>(Mg * H);
    L.GBp = c.take<char>(Mu * I * es);
    L.dXu = c.take<float>(Mu * H);
    if (gl) {
      L.xrow_g = c.take<int32_t>(Mg);
      L.xw_g = c.take<float>(Mg);
      L.xrow_u = c.take<int32_t>(Mu);
      L.xw_u = c.take<float>(Mu);
    } else {
      L.Xg = c.take<char>(Mg * H * es);
      L.Xu = c.take<char>(Mu * H * es);
    }
  }
  if (out) {
    if (out->score) L.score = out->score;
    if (out->pos) L.pos = out->pos;
    if (out->offsets) L.offsets = out->offsets;
    if (out->score_gate) L.s_gate = out->score_gate;
    if (out->score_up) L.s_up = out->score_up;
    if (out->pos_gate) L.pos_g = out->pos_gate;
    if (out->pos_up) L.pos_u = out->pos_up;
    if (out->offsets_gate) L.off_g = out->offsets_gate;
    if (out->offsets_up) L.off_u = out->offsets_up;
    if (out->dH) L.U = out->dH;
  }
  return L;
}

// Sizes the host can fix from the quotas (no device sync).
struct GluSizes {
  int64_t Md, Mg, Mu;
  bool pass_through;
};

GluSizes glu_sizes(const lrm_problem* pb) {
  const int N = pb->pairs.N, E = pb->pairs.E;
  GluSizes z{};
  if (pb->flags & LRM_KEEP_ALL) {
    z.Md = z.Mg = z.Mu = N;
    z.pass_through = true;
    return z;
  }
  if (pb->flags & LRM_QUOTA_ON_DEVICE) {  // quotas the host cannot read
    z.Md = z.Mg = z.Mu = N;
    z.pass_through = false;
    return z;
  }
  z.Md = lrm_max_kept(N, E, pb->quota_down);
  z.Mg = lrm_max_kept((int32_t)z.Md, E, pb->quota_gate);
  z.Mu = lrm_max_kept((int32_t)z.Md, E, pb->quota_up);
  // the gate/up selections keep everything the down stage kept when their
  // quotas are at least the down quotas (M_down,e <= q_down,e)
  bool pt = true;
  for (int e = 0; e < E; ++e)
    pt = pt && pb->quota_gate[e] >= pb->quota_down[e] && pb->quota_up[e] >= pb->quota_down[e];
  z.pass_through = pt;
  return z;
}

lrm_status check_problem(const lrm_problem* pb, const lrm_outputs* out) {
  if (!pb) return LRM_ERR_NULL;
  LRM_TRY(check_pairs(&pb->pairs));
  if (pb->flags & ~(LRM_KEEP_ALL | LRM_DW_BF16 | LRM_QUOTA_ON_DEVICE | LRM_DEBUG_CHECKS |
                    LRM_GATHER_LOADS))
    return LRM_ERR_UNSUPPORTED;
  if (pb->dtype != LRM_F32 && pb->dtype != LRM_BF16) return LRM_ERR_DTYPE;
  if ((pb->flags & LRM_DW_BF16) && pb->dtype != LRM_BF16) return LRM_ERR_UNSUPPORTED;
  const lrm_pairs* p = &pb->pairs;
  const bool keep_all = (pb->flags & LRM_KEEP_ALL) != 0;
  const bool qdev = (pb->flags & LRM_QUOTA_ON_DEVICE) != 0;
  // host quotas are checked (non-negative); device quotas only for presence
  auto check_q = [&](const int32_t* q) {
    return qdev ? (q ? LRM_OK : LRM_ERR_NULL) : check_quota(q, p->E, nullptr);
  };
  const int q = 16 / esize(pb->dtype);
  if (pb->kind == LRM_LINEAR) {
    if (pb->d_in <= 0 || pb->d_out <= 0 || pb->d_in > kMaxDim || pb->d_out > kMaxDim)
      return LRM_ERR_SHAPE;
    LRM_TRY(check_mat(&pb->X, p, pb->dtype, pb->d_in, -1));
    LRM_TRY(check_mat(&pb->G, p, pb->dtype, pb->d_out, -1));
    if (p->E > 0 && !pb->W) return LRM_ERR_NULL;
    if (!aligned16(pb->W)) return LRM_ERR_ALIGN;
    if (pb->w_stride < (int64_t)pb->d_in * pb->d_out) return LRM_ERR_SHAPE;
    if ((pb->w_stride * esize(pb->dtype)) % 16) return LRM_ERR_ALIGN;
    if (!keep_all) LRM_TRY(check_q(pb->quota));
  } else if (pb->kind == LRM_SWIGLU) {
    if (pb->H <= 0 || pb->I <= 0 || pb->H > kMaxDim || pb->I > kMaxDim) return LRM_ERR_SHAPE;
    if (pb->H % q || pb->I % q) return LRM_ERR_UNSUPPORTED;
    LRM_TRY(check_mat(&pb->X, p, pb->dtype, pb->H, LRM_ROWS_TOKEN));
    LRM_TRY(check_mat(&pb->G, p, pb->dtype, pb->H, LRM_ROWS_TOKEN));
    LRM_TRY(check_mat(&pb->A, p, pb->dtype, pb->I, LRM_ROWS_PAIR));
    LRM_TRY(check_mat(&pb->B, p, pb->dtype, pb->I, LRM_ROWS_PAIR));
    if (!pb->W_gate || !pb->W_up || !pb->W_down) return LRM_ERR_NULL;
    if (!aligned16(pb->W_gate) || !aligned16(pb->W_up) || !aligned16(pb->W_down))
      return LRM_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(pb->h_sumsq) & 7u) != 0) return LRM_ERR_ALIGN;
    if (!keep_all) {
      LRM_TRY(check_q(pb->quota_down));
      LRM_TRY(check_q(pb->quota_gate));
      LRM_TRY(check_q(pb->quota_up));
    }
  } else {
    return LRM_ERR_UNSUPPORTED;
  }
  if (out) {
    const int64_t xrows = pb->X.rows == LRM_ROWS_TOKEN ? p->T : p->N;
    if (xrows > 0 && !out->dX) return LRM_ERR_NULL;
    if (!aligned16(out->dX)) return LRM_ERR_ALIGN;
    if (pb->kind == LRM_LINEAR) {
      if (!out->dW) return LRM_ERR_NULL;
      if (!aligned16(out->dW)) return LRM_ERR_ALIGN;
    } else {
      if (!out->dW_gate || !out->dW_up || !out->dW_down) return LRM_ERR_NULL;
      if (!aligned16(out->dW_gate) || !aligned16(out->dW_up) || !aligned16(out->dW_down))
        return LRM_ERR_ALIGN;
    }
  }
  return LRM_OK;
}

size_t plan_size(const lrm_problem* pb, const lrm_outputs* out) {
  Carve c(nullptr);
  if (pb->kind == LRM_LINEAR) {
    const int64_t Mcap = (pb->flags & (LRM_KEEP_ALL | LRM_QUOTA_ON_DEVICE))
                             ? pb->pairs.N
                             : lrm_max_kept(pb->pairs.N, pb->pairs.E, pb->quota);
    carve_linear(c, pb, out, Mcap);
  } else {
    GluSizes z = glu_sizes(pb);
    carve_glu(c, pb, out, z.Md, z.Mg, z.Mu, z.pass_through);
  }
  return c.size();
}

// Optional profiling events recorded at stage boundaries.
struct Marks {
  void* const* ev;
  int n;
  hipStream_t s;
  hipError_t operator()(int i) const {
    if (ev && i < n && ev[i]) return hipEventRecord(reinterpret_cast<hipEvent_t>(ev[i]), s);
    return hipSuccess;
  }
  // the event of boundary i, for a launcher to record inside its sequence
  hipEvent_t at(int i) const {
    return ev && i < n ? reinterpret_cast<hipEvent_t>(ev[i]) : nullptr;
  }
};

lrm_status run_linear(const lrm_problem* pb, const lrm_outputs* out, void* ws, hipStream_t s,
                      const Marks& mark) {
  const lrm_pairs* p = &pb->pairs;
  const bool keep_all = (pb->flags & LRM_KEEP_ALL) != 0;
  const bool qdev = (pb->flags & LRM_QUOTA_ON_DEVICE) != 0;
  const int64_t Mcap = keep_all || qdev ? p->N : lrm_max_kept(p->N, p->E, pb->quota);
  Carve c(ws);
  LinearPlan L = carve_linear(c, pb, out, Mcap);
  const int bf16 = pb->dtype == LRM_BF16;
  // the grouped GEMM's launch shape (its dX row-tile prefix is built by the
  // selection pass)
  GemmArgs g{};
  g.E = p->E; g.bf16 = bf16; g.max_rows = (int)Mcap;
  const int dx_rows = gemm_dx_tile_rows(g);
  LRM_TRY_HIP(mark(0));
  // 1. LRM score of every pair
  if (!keep_all) LRM_TRY_HIP(run_score(p, &pb->X, &pb->G, L.score, L.sc, s));
  LRM_TRY_HIP(mark(1));
  // 2. per-expert top-quota selection and packed rows
  // (the token offsets of the unpermute step come out of the bucketing pass)
  const bool tok_out = pb->X.rows != LRM_ROWS_PAIR;
  LRM_TRY(run_select(p, L.score, keep_all ? nullptr : pb->quota, L.pos, L.offsets, L.kept,
                     L.sel, s, tok_out && p->N > 0 ? L.tok_off : nullptr, L.mt_off, dx_rows,
                     qdev, Mcap));
  LRM_TRY_HIP(mark(2));
  // 3. compaction: Xp = w x, Gp = g
  CompactArgs ca{};
  ca.T = p->T; ca.bf16 = bf16; ca.max_rows = (int)Mcap; ca.E = p->E;
  ca.offsets = L.offsets; ca.kept = L.kept; ca.token = p->token; ca.weight = p->weight;
  ca.X = pb->X.ptr; ca.ldx = pb->X.ld; ca.xcols = pb->d_in;
  ca.x_pair = pb->X.rows == LRM_ROWS_PAIR; ca.Xp = L.Xp;
  ca.G = pb->G.ptr; ca.ldg = pb->G.ld; ca.gcols = pb->d_out;
  ca.g_pair = pb->G.rows == LRM_ROWS_PAIR; ca.Gp = L.Gp;
  if (L.xrow) {  // the dW loader gathers w x itself: pack g, map the x rows
    ca.Xp = nullptr;
    LRM_TRY_HIP(launch_row_map(ca, L.xrow, L.xw, s));
  }
  LRM_TRY_HIP(launch_compact(ca, s));
  LRM_TRY_HIP(mark(3));
  // 4. grouped GEMM: dW_e = Gp_e^T Xp_e, dXp_e = Gp_e W_e
  g.d_in = pb->d_in; g.d_out = pb->d_out;
  g.offsets = L.offsets; g.Gp = L.Gp; g.Xp = L.Xp; g.W = pb->W; g.w_stride = pb->w_stride;
  g.dW = out->dW; g.dXp = L.dXp; g.mt_off = L.mt_off; g.mt_ready = 1;
  g.dw_bf16 = (pb->flags & LRM_DW_BF16) != 0;
  if (L.xrow) {
    g.xrow = L.xrow; g.xw = L.xw; g.xsrc = pb->X.ptr; g.ldxs = pb->X.ld;
    g.xsrc_rows = pb->X.rows == LRM_ROWS_PAIR ? p->N : p->T;
  }
  g.mid_event = mark.at(4);
  LRM_TRY_HIP(launch_grouped_gemm(g, s));
  LRM_TRY_HIP(mark(5));
  // 5. back to the layout of X, times the routing weight
  ScatterArgs sa{};
  sa.N = p->N; sa.T = p->T; sa.d = pb->d_in; sa.out_pair = pb->X.rows == LRM_ROWS_PAIR;
  sa.token = p->token; sa.weight = p->weight; sa.pos[0] = L.pos; sa.src[0] = L.dXp;
  sa.src_rows[0] = (int)Mcap;
  if (!sa.out_pair) {
    if (p->N == 0) LRM_TRY_HIP(launch_token_offsets(p->N, p->T, p->token, L.tok_off, s));
    sa.tok_off = L.tok_off;
  }
  sa.dX = out->dX;
  LRM_TRY_HIP(launch_unpermute(sa, s));
  LRM_TRY_HIP(mark(6));
  return LRM_OK;
}

lrm_status run_swiglu(const lrm_problem* pb, const lrm_outputs* out, void* ws, hipStream_t s,
                      const Marks& mark) {
  const lrm_pairs* p = &pb->pairs;
  const bool keep_all = (pb->flags & LRM_KEEP_ALL) != 0;
  const GluSizes z = glu_sizes(pb);
  Carve c(ws);
  GluPlan L = carve_glu(c, pb, out, z.Md, z.Mg, z.Mu, z.pass_through);
  const int bf16 = pb->dtype == LRM_BF16;
  const int H = pb->H, I = pb->I, E = p->E;
  // Gate and up keep the same rows (one packing): their weight gradients are
  // one product Gp^T X with Gp = [GA | GB] ([rows][2I], the SwiGLU backward
  // writes GA and GB side by side into the span of both) split over dW_gate
  // and dW_up, which tiles 2I where I alone leaves a part-filled last tile.
  // bf16 kernels, I a multiple of 64 (the split falls between waves), packed
  // w x (the gathering loaders write one output).
  // (LRM_FUSE_GATE_UP=0 keeps two launches, for comparison.)
  const char* fenv = getenv("LRM_FUSE_GATE_UP");
  const bool fuse_gu = z.pass_through && bf16 && I % 64 == 0 && !L.xrow_g &&
                       !(fenv && fenv[0] == '0');
  void* const GBw = fuse_gu ? static_cast<void*>(static_cast<char*>(L.GA) + (int64_t)I * 2) : L.GB;
  // the one gate/up weight-gradient launch: its schedule depends only on the
  // down stage's offsets, so the down launch's plan launch writes it as well
  GemmArgs gw{};
  gw.E = E; gw.bf16 = bf16; gw.max_rows = (int)z.Md; gw.d_in = H; gw.d_out = 2 * I;
  gw.offsets = L.offsets; gw.Gp = L.GA; gw.Xp = L.Xgu;
  gw.dW = out->dW_gate; gw.dW2 = out->dW_up; gw.dw_split = I;
  gw.mt_off = L.mt_off2; gw.dw_plan_ready = 1;
  gw.dw_bf16 = (pb->flags & LRM_DW_BF16) != 0;
  GemmArgs gd{};
  gd.E = E; gd.bf16 = bf16; gd.max_rows = (int)z.Md;
  const int dx_rows = gemm_dx_tile_rows(gd);
  LRM_TRY_HIP(mark(0));
  // ---- down projection: input h = silu(a) * b, gradient g = G row
  if (!keep_all)
    LRM_TRY_HIP(run_score_glu(p, &pb->A, &pb->B, &pb->G, L.score, L.sc, s, pb->h_sumsq));
  LRM_TRY_HIP(mark(1));
  // (the token offsets of the unpermute step come out of the bucketing pass)
  const bool tok_out = pb->X.rows != LRM_ROWS_PAIR;
  const bool qdev = (pb->flags & LRM_QUOTA_ON_DEVICE) != 0;
  LRM_TRY(run_select(p, L.score, keep_all ? nullptr : pb->quota_down, L.pos, L.offsets, L.kept,
                     L.sel, s, tok_out && p->N > 0 ? L.tok_off : nullptr, L.mt_off, dx_rows,
                     qdev, z.Md));
  LRM_TRY_HIP(mark(2));
  CompactArgs cd{};
  cd.T = p->T; cd.bf16 = bf16; cd.max_rows = (int)z.Md; cd.E = E;
  cd.offsets = L.offsets; cd.kept = L.kept; cd.token = p->token; cd.weight = p->weight;
  cd.glu = 1; cd.X = pb->A.ptr; cd.ldx = pb->A.ld; cd.X2 = pb->B.ptr; cd.ldx2 = pb->B.ld;
  cd.xcols = I; cd.x_pair = 1; cd.Xp = L.Hd;
  cd.G = pb->G.ptr; cd.ldg = pb->G.ld; cd.gcols = H; cd.g_pair = pb->G.rows == LRM_ROWS_PAIR;
  cd.Gp = L.Gd;
  LRM_TRY_HIP(launch_compact(cd, s));
  LRM_TRY_HIP(mark(3));
  gd.d_in = I; gd.d_out = H;
  gd.offsets = L.offsets; gd.Gp = L.Gd; gd.Xp = L.Hd;
  gd.W = pb->W_down; gd.w_stride = (int64_t)H * I;
  gd.dW = out->dW_down; gd.dXp = L.U; gd.mt_off = L.mt_off; gd.mt_ready = 1;
  gd.dw_bf16 = (pb->flags & LRM_DW_BF16) != 0;
  gd.mid_event = mark.at(4);
  gd.dw_plan_next = fuse_gu ? &gw : nullptr;
  LRM_TRY_HIP(launch_grouped_gemm(gd, s));
  LRM_TRY_HIP(mark(5));
  // ---- SwiGLU backward and the gate/up scores
  const bool x_pair = pb->X.rows == LRM_ROWS_PAIR;
  if (!keep_all)
    LRM_TRY_HIP(launch_row_sumsq(pb->X.ptr, bf16, pb->X.ld, H, x_pair ? p->N : p->T, L.x2, s));
  GluBwdArgs gb{};
  gb.T = p->T; gb.bf16 = bf16; gb.max_rows = (int)z.Md; gb.E = E; gb.I = I;
  gb.offsets_down = L.offsets; gb.kept_down = L.kept; gb.token = p->token; gb.weight = p->weight;
  gb.U = L.U; gb.A = pb->A.ptr; gb.lda = pb->A.ld; gb.B = pb->B.ptr; gb.ldb = pb->B.ld;
  gb.x2 = L.x2; gb.x_pair = x_pair; gb.GA = L.GA; gb.GB = GBw; gb.ldg = fuse_gu ? 2 * I : 0;
  gb.s_gate = keep_all ? nullptr : L.s_gate;
  gb.s_up = keep_all ? nullptr : L.s_up;
  LRM_TRY_HIP(launch_glu_bwd(gb, s));
  LRM_TRY_HIP(mark(6));
  // ---- gate/up selections among the down-kept rows (candidate ids = rows)
  if (!keep_all) {
    // quotas: device arrays, by value (host, E <= kQuotaPackMax), or copied
    const int32_t* qg = pb->quota_gate;
    const int32_t* qu = pb->quota_up;
    QuotaPack pg, pu;
    const bool by_value = !qdev && E <= kQuotaPackMax;
    if (by_value) {
      std::memcpy(pg.q, pb->quota_gate, sizeof(int32_t) * E);
      std::memcpy(pu.q, pb->quota_up, sizeof(int32_t) * E);
      qg = qu = nullptr;
    } else if (!qdev) {
      LRM_TRY_HIP(hipMemcpyAsync(L.qgate, pb->quota_gate, sizeof(int32_t) * E,
                                 hipMemcpyHostToDevice, s));
      LRM_TRY_HIP(hipMemcpyAsync(L.qup, pb->quota_up, sizeof(int32_t) * E,
                                 hipMemcpyHostToDevice, s));
      qg = L.qgate;
      qu = L.qup;
    }
    // candidates are down rows: the per-row arrays hold Md of them
    LRM_TRY_HIP(launch_kept_offsets(E, L.offsets, qg, by_value ? &pg : nullptr, L.off_g,
                                    L.sel.err, z.Mg, s));
    LRM_TRY_HIP(launch_select(E, L.offsets, L.off_g,
                              reinterpret_cast<const uint32_t*>(L.s_gate), nullptr, L.pos_g,
                              L.kept_g, (int)z.Md, s));
    LRM_TRY_HIP(launch_kept_offsets(E, L.offsets, qu, by_value ? &pu : nullptr, L.off_u,
                                    L.sel.err, z.Mu, s));
    LRM_TRY_HIP(launch_select(E, L.offsets, L.off_u, reinterpret_cast<const uint32_t*>(L.s_up),
                              nullptr, L.pos_u, L.kept_u, (int)z.Md, s));
  }
  LRM_TRY_HIP(mark(7));
  const bool x_tok = !x_pair;
  ScatterArgs sa{};
  sa.N = p->N; sa.T = p->T; sa.d = H; sa.out_pair = x_pair;
  sa.token = p->token; sa.weight = p->weight;
  if (z.pass_through) {
    // both selections keep every down-kept row: one packing, and the two
    // input-gradient products share one GEMM with K = 2I
    CompactArgs cx{};
    cx.T = p->T; cx.bf16 = bf16; cx.max_rows = (int)z.Md; cx.E = E;
    cx.offsets = L.offsets; cx.kept = L.kept; cx.token = p->token; cx.weight = p->weight;
    cx.X = pb->X.ptr; cx.ldx = pb->X.ld; cx.xcols = H; cx.x_pair = x_pair; cx.Xp = L.Xgu;
    if (L.xrow_g)  // the gate/up dW loaders gather w x: map the rows only
      LRM_TRY_HIP(launch_row_map(cx, L.xrow_g, L.xw_g, s));
    else
      LRM_TRY_HIP(launch_compact(cx, s));
    LRM_TRY_HIP(mark(8));
    if (fuse_gu) {
      LRM_TRY_HIP(launch_grouped_gemm(gw, s));
      LRM_TRY_HIP(mark(9));
      // both input-gradient products, K = 2I in two segments of [GA | GB]
      GemmArgs gx{};
      gx.E = E; gx.bf16 = bf16; gx.max_rows = (int)z.Md; gx.d_in = H; gx.d_out = I;
      gx.lda = 2 * I;
      gx.offsets = L.offsets; gx.Gp = L.GA; gx.W = pb->W_gate; gx.w_stride = (int64_t)I * H;
      gx.Gp2 = GBw; gx.W2 = pb->W_up; gx.w2_stride = (int64_t)I * H; gx.d_out2 = I;
      gx.dXp = L.dXp; gx.mt_off = L.mt_off;
      LRM_TRY_HIP(launch_grouped_gemm(gx, s));
      LRM_TRY_HIP(mark(10));
      LRM_TRY_HIP(mark(11));
      LRM_TRY_HIP(mark(12));
      sa.pos[0] = L.pos; sa.src[0] = L.dXp; sa.src_rows[0] = (int)z.Md;
    } else {
      GemmArgs gg{};
      gg.E = E; gg.bf16 = bf16; gg.max_rows = (int)z.Md; gg.d_in = H; gg.d_out = I;
      gg.offsets = L.offsets; gg.Gp = L.GA; gg.Xp = L.Xgu;
      gg.W = pb->W_gate; gg.w_stride = (int64_t)I * H;
      gg.Gp2 = L.GB; gg.W2 = pb->W_up; gg.w2_stride = (int64_t)I * H; gg.d_out2 = I;
      gg.dW = out->dW_gate; gg.dXp = L.dXp; gg.mt_off = L.mt_off;
      gg.dw_bf16 = (pb->flags & LRM_DW_BF16) != 0;
      const int64_t xsrc_rows = x_pair ? p->N : p->T;
      if (L.xrow_g) {
        gg.xrow = L.xrow_g; gg.xw = L.xw_g; gg.xsrc = pb->X.ptr; gg.ldxs = pb->X.ld;
        gg.xsrc_rows = xsrc_rows;
      }
      gg.mid_event = mark.at(9);
      // the down projection's dW launch left the schedule of these offsets and
      // max_rows in the workspace: the gate and up launches reuse it when their
      // tiles per expert agree (the schedule depends on nothing else)
      const int plan_per = gemm_dw_tiles_per_expert(gd);
      gg.dw_plan_ready = plan_per > 0 && gemm_dw_tiles_per_expert(gg) == plan_per;
      LRM_TRY_HIP(launch_grouped_gemm(gg, s));
      LRM_TRY_HIP(mark(10));
      GemmArgs gu{};
      gu.E = E; gu.bf16 = bf16; gu.max_rows = (int)z.Md; gu.d_in = H; gu.d_out = I;
      gu.offsets = L.offsets; gu.Gp = L.GB; gu.Xp = L.Xgu;
      gu.dW = out->dW_up; gu.dXp = nullptr; gu.mt_off = L.mt_off;
      gu.dw_bf16 = (pb->flags & LRM_DW_BF16) != 0;
      gu.dw_plan_ready = plan_per > 0 && gemm_dw_tiles_per_expert(gu) == plan_per;
      if (L.xrow_u) {
        gu.xrow = L.xrow_u; gu.xw = L.xw_u; gu.xsrc = pb->X.ptr; gu.ldxs = pb->X.ld;
        gu.xsrc_rows = xsrc_rows;
      }
      LRM_TRY_HIP(launch_grouped_gemm(gu, s));
      LRM_TRY_HIP(mark(11));
      LRM_TRY_HIP(mark(12));
      sa.pos[0] = L.pos; sa.src[0] = L.dXp; sa.src_rows[0] = (int)z.Md;
    }
  } else {
    const void* GAsrc[2] = {L.GA, L.GB};
    int32_t* keptv[2] = {L.kept_g, L.kept_u};
    int32_t* offv[2] = {L.off_g, L.off_u};
    void* Gpv[2] = {L.GAp, L.GBp};
    void* Xpv[2] = {L.Xg, L.Xu};
    float* dXv[2] = {L.dXg, L.dXu};
    const void* Wv[2] = {pb->W_gate, pb->W_up};
    float* dWv[2] = {out->dW_gate, out->dW_up};
    const int64_t cap[2] = {z.Mg, z.Mu};
    int32_t* posv[2] = {L.pos_g, L.pos_u};
    int32_t* xrowv[2] = {L.xrow_g, L.xrow_u};
    float* xwv[2] = {L.xw_g, L.xw_u};
    for (int k = 0; k < 2; ++k) {
      CompactArgs cg{};
      cg.T = p->T; cg.bf16 = bf16; cg.max_rows = (int)cap[k]; cg.E = E;
      cg.offsets = offv[k]; cg.kept = keptv[k]; cg.pairmap = L.kept;
      cg.token = p->token; cg.weight = p->weight;
      cg.X = pb->X.ptr; cg.ldx = pb->X.ld; cg.xcols = H; cg.x_pair = x_pair; cg.Xp = Xpv[k];
      cg.G = GAsrc[k]; cg.ldg = I; cg.gcols = I; cg.g_by_id = 1; cg.Gp = Gpv[k];
      if (xrowv[k]) {  // the dW loader gathers w x: map the rows, pack g only
        LRM_TRY_HIP(launch_row_map(cg, xrowv[k], xwv[k], s));
        cg.Xp = nullptr;
      }
      LRM_TRY_HIP(launch_compact(cg, s));
    }
    LRM_TRY_HIP(mark(8));
    for (int k = 0; k < 2; ++k) {
      GemmArgs gk{};
      gk.E = E; gk.bf16 = bf16; gk.max_rows = (int)cap[k]; gk.d_in = H; gk.d_out = I;
      gk.offsets = offv[k]; gk.Gp = Gpv[k]; gk.Xp = Xpv[k];
      gk.W = Wv[k]; gk.w_stride = (int64_t)I * H;
      gk.dW = dWv[k]; gk.dXp = dXv[k]; gk.mt_off = L.mt_off;
      gk.dw_bf16 = (pb->flags & LRM_DW_BF16) != 0;
      if (xrowv[k]) {
        gk.xrow = xrowv[k]; gk.xw = xwv[k]; gk.xsrc = pb->X.ptr; gk.ldxs = pb->X.ld;
        gk.xsrc_rows = x_pair ? p->N : p->T;
      }
      gk.mid_event = mark.at(9 + 2 * k);
      LRM_TRY_HIP(launch_grouped_gemm(gk, s));
      LRM_TRY_HIP(mark(10 + 2 * k));
      sa.pos[k] = L.pos; sa.pos2[k] = posv[k]; sa.src[k] = dXv[k];
      sa.pos2_rows[k] = (int)z.Md; sa.src_rows[k] = (int)cap[k];
    }
  }
  if (x_tok) {
    if (p->N == 0) LRM_TRY_HIP(launch_token_offsets(p->N, p->T, p->token, L.tok_off, s));
    sa.tok_off = L.tok_off;
  }
  sa.dX = out->dX;
  LRM_TRY_HIP(launch_unpermute(sa, s));
  LRM_TRY_HIP(mark(13));
  return LRM_OK;
}

}  // namespace

extern "C" {

size_t lrm_workspace_size(const lrm_problem* prob) {
  if (check_problem(prob, nullptr) != LRM_OK) return 0;
  return plan_size(prob, nullptr);
}

lrm_status lrm_expert_backward_events(const lrm_problem* prob, const lrm_outputs* out, void* ws,
                                      size_t ws_bytes, void* stream, void* const* events,
                                      int32_t n_events) {
  if (!out) return LRM_ERR_NULL;
  LRM_TRY(check_problem(prob, out));
  if (!ws || ws_bytes < plan_size(prob, out)) return LRM_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return LRM_ERR_ALIGN;
  hipStream_t s = as_stream(stream);
  LRM_TRY(check_capturable(prob->pairs.E,
                           !(prob->flags & (LRM_KEEP_ALL | LRM_QUOTA_ON_DEVICE)), s));
  const Marks mark{events, n_events, s};
  LRM_TRY(prob->kind == LRM_LINEAR ? run_linear(prob, out, ws, s, mark)
                                   : run_swiglu(prob, out, ws, s, mark));
  if (prob->flags & LRM_DEBUG_CHECKS) return lrm_check_device_errors(ws, stream);
  return LRM_OK;
}

lrm_status lrm_expert_backward(const lrm_problem* prob, const lrm_outputs* out, void* ws,
                               size_t ws_bytes, void* stream) {
  return lrm_expert_backward_events(prob, out, ws, ws_bytes, stream, nullptr, 0);
}

}  // extern "C"

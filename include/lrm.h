/*
 * lrm.h -- C ABI of the LRM-pruned MoE expert backward for one GPU's share of
 * the experts (gfx950 / MI355X, HIP).
 *
 * The method (LRMoE, "load recalibration"): the forward stays complete; a
 * controller fixes, per expert, how many token->expert pairs are kept in the
 * backward for the whole layer call; when the gradient reaches the layer every
 * pair is scored by the LRM metric, the squared Frobenius norm of its
 * weight-gradient contribution, which factorises as
 *     score = w^2 * |g|^2 * |x|^2
 * (w routing weight, g incoming gradient at the projection output, x saved
 * projection input); the top-quota pairs of each expert are kept, their rows
 * are packed into dense per-expert blocks, the expert products run as
 * variable-size grouped GEMMs without zero padding and the result is returned
 * to the original layout.
 *
 * Sources: the page "LRMoE урезает обратный проход MoE и ускоряет обучение на
 * 21–45%" (news.hamidun.com), section "Что делает LRMoE: полный прямой
 * проход, обрезанный обратный", bullets "Квоты до вычислений" (quotas),
 * "Отбор по метрике LRM" (scoring and selection) and "Физическое уплотнение"
 * (compaction, grouped GEMM, return to layout), and the note after them on
 * masking; its French twin "LRMoE élague la passe arrière des MoE ..." (same
 * section); the German summary "LRMoE führt eine Nachkalibrierung der Last
 * ... ein" (ai.mistergeeks.com), paragraph on the Lastnachkalibrierungs-
 * Metrik.  Readings where the pages are silent:
 *   - g is unscaled; the routing weight enters the contribution as w g x^T;
 *   - ties in score are broken by lower pair index;
 *   - a dropped pair contributes to neither dW nor dX;
 *   - SwiGLU runs down -> gate/up; the gate/up candidates of an expert are the
 *     pairs its down stage kept; each projection has its own score and quota.
 *
 * Conventions common to every call:
 *   - Every pointer argument is caller-owned.  Pointers documented "device"
 *     must be device memory of the current HIP device; "host" ones host memory.
 *     The library never allocates or frees memory.
 *   - Calls are asynchronous on the given stream (a hipStream_t passed as
 *     void*, NULL = default stream) unless documented otherwise.  Host-side
 *     argument validation happens before any launch: a call that returns an
 *     error other than LRM_ERR_HIP has enqueued nothing and touched no memory.
 *   - Pairs are indexed p = 0..N-1, token-major: token[] is non-decreasing.
 *     N, T, E are pairs, tokens and experts resident on this GPU.
 *   - Dense inputs are row-major with a leading dimension ld (elements) and
 *     16-byte aligned rows; all dense inputs of one call share one dtype;
 *     columns must be a multiple of 8 (bf16) or 4 (fp32).  Outputs are fp32.
 *   - Outputs are overwritten, never accumulated.  Experts with nothing kept
 *     get dW = 0; rows of dX that receive no kept pair are 0.
 *   - Inputs must be finite; otherwise the results are undefined.
 *   - Every call is deterministic: the same inputs give bit-identical outputs
 *     (no floating-point atomics; all reductions in a fixed order).
 *   - No exception crosses this interface.  Functions are re-entrant when
 *     concurrent calls use distinct workspaces and outputs.
 *   - Environment variables read at each call, for benchmarking and testing
 *     (the defaults are the tuned paths): LRM_GEMM_TILE=S|M|L|X forces one
 *     bf16 tile configuration of the grouped GEMM; LRM_GEMM_DMA=2|4 runs the
 *     256x256 tiles with operands loaded straight into LDS (bit-identical
 *     results, slower on the measured shapes); LRM_SELECT_ONE_LAUNCH=0 keeps
 *     calls of up to 8192 pairs on the bucketing kernels (bit-identical
 *     results); LRM_FUSE_GATE_UP=0 runs the SwiGLU gate and up weight
 *     gradients as two launches where one would compute both (bit-identical
 *     results under the same tile configuration).  Workspace sizes do not
 *     depend on them.
 */
#ifndef LRM_H_
#define LRM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lrm_status {
  LRM_OK = 0,
  LRM_ERR_NULL = 1,        /* a required pointer is NULL */
  LRM_ERR_SHAPE = 2,       /* sizes inconsistent or out of the supported range */
  LRM_ERR_DTYPE = 3,       /* unknown dtype, or dense inputs of mixed dtype */
  LRM_ERR_LAYOUT = 4,      /* unknown row layout, or a layout this call does not take */
  LRM_ERR_ALIGN = 5,       /* a pointer or leading dimension breaks 16-byte row alignment */
  LRM_ERR_QUOTA = 6,       /* a negative quota */
  LRM_ERR_WORKSPACE = 7,   /* workspace NULL or smaller than required */
  LRM_ERR_INDEX = 8,       /* device-detected: expert or token index out of range / order,
                              or a replica assignment that does not match the kept counts */
  LRM_ERR_HIP = 9,         /* a HIP runtime call or kernel launch failed */
  LRM_ERR_UNSUPPORTED = 10, /* valid request outside what this library implements */
  LRM_ERR_INFEASIBLE = 11  /* kept pairs that no replica (or no capacity) can take */
} lrm_status;

typedef enum lrm_dtype { LRM_F32 = 0, LRM_BF16 = 1 } lrm_dtype;

/* Which row of a matrix a pair p reads: row token[p] (one row per token, shared
 * by the token's pairs) or row p (one row per pair). */
typedef enum lrm_rows { LRM_ROWS_TOKEN = 0, LRM_ROWS_PAIR = 1 } lrm_rows;

typedef enum lrm_kind { LRM_LINEAR = 0, LRM_SWIGLU = 1 } lrm_kind;

/* Flags of lrm_expert_backward. */
#define LRM_KEEP_ALL 1u /* unpruned baseline: every pair kept, no score/select */
/* Weight gradients stored as bf16: dW (or dW_gate, dW_up, dW_down) point to
 * bf16 arrays of the same shape, each element the fp32 result rounded to
 * nearest even (accumulation stays fp32; the other outputs are unchanged).
 * Halves the dW bytes, which are fixed per expert and dominate when few pairs
 * are kept.  bf16 inputs only (LRM_ERR_UNSUPPORTED otherwise). */
#define LRM_DW_BF16 2u
/* Quotas in device memory: quota (lrm_select, the LINEAR problem) and
 * quota_down, quota_gate, quota_up (SWIGLU) are device pointers to int32[E],
 * read by the kernels in stream order, never by the host (a controller on the
 * GPU can write them just before the call).  The host then cannot size the
 * packed blocks from the quotas: lrm_workspace_size assumes every pair kept,
 * and a SWIGLU call always runs its gate/up selections (the one-packing path
 * for gate/up quotas at least the down quotas needs the host to compare them).
 * Negative quotas cannot be checked on the host and keep nothing.  Results are
 * the same as with the same quotas on the host. */
#define LRM_QUOTA_ON_DEVICE 4u
/* Debug checks: lrm_expert_backward synchronises its stream at the end and
 * returns LRM_ERR_INDEX if a kernel of the call found an expert id or token
 * out of range, or tokens out of order (what lrm_check_device_errors reports,
 * and clears, without the extra call). */
#define LRM_DEBUG_CHECKS 8u
/* Gathering GEMM loaders (bf16 inputs): the weight-gradient GEMMs whose
 * packed operand is w * x (LINEAR; the SwiGLU gate and up projections) read
 * the kept rows of X themselves, scaling them by w and rounding to bf16 in
 * the loader, instead of reading a packed copy that compaction writes; the
 * compaction then writes only a row map (4 + 4 bytes per kept row).  Results
 * are bit for bit those of the call without the flag.  Trades time for
 * memory: the workspace loses the packed copy (kept rows x d_in x 2 bytes),
 * but the gathering loaders are slower than the packed ones on MI355X.
 * Ignored for fp32 inputs and when X takes 2 GiB or more. */
#define LRM_GATHER_LOADS 16u

/* The routed pairs of one layer call (the page's "pair": one token -> expert
 * choice; page 1 introduction). */
typedef struct lrm_pairs {
  int32_t T;             /* tokens (rows of TOKEN-layout matrices), >= 0 */
  int32_t N;             /* pairs resident on this GPU, >= 0 */
  int32_t E;             /* experts resident on this GPU, 1..4096 */
  int32_t _pad;
  const int32_t* token;  /* device [N], non-decreasing, in [0, T) */
  const int32_t* expert; /* device [N], in [0, E) */
  const float* weight;   /* device [N], routing weight w_p */
} lrm_pairs;

/* A dense matrix whose rows are addressed through the pairs. */
typedef struct lrm_mat {
  const void* ptr; /* device, row-major */
  int32_t dtype;   /* lrm_dtype */
  int32_t rows;    /* lrm_rows: T rows (TOKEN) or N rows (PAIR) */
  int32_t cols;
  int32_t _pad;
  int64_t ld;      /* elements between consecutive rows, >= cols */
} lrm_mat;

/* ------------------------------------------------------------------ steps */

/* LRM score of every pair (page 1, bullet "Отбор по метрике LRM"):
 *   score[p] = w_p^2 * |G row of p|^2 * |X row of p|^2
 * Row sums of squares are accumulated in fp64 and the product is formed in
 * fp64, then rounded to the nearest fp32 (scores are >= 0, so their fp32 bit
 * patterns order like the values).  Each TOKEN-layout matrix is read once per
 * token, each PAIR-layout matrix once per pair.
 * score: device [N] fp32 output.  ws: device scratch of at least
 * lrm_score_workspace_size(pairs) bytes (fp64 per-token norms). */
lrm_status lrm_score(const lrm_pairs* pairs, const lrm_mat* X, const lrm_mat* G, float* score,
                     void* ws, size_t ws_bytes, void* stream);
size_t lrm_score_workspace_size(const lrm_pairs* pairs);

/* LRM score of the down projection of a SwiGLU expert, whose saved input
 * h_p = silu(a_p) * b_p is formed on the fly from the saved gate/up
 * pre-activations A, B (PAIR layout, I columns) and whose incoming gradient is
 * the G row of p (TOKEN or PAIR, H columns):
 *   score[p] = w_p^2 * |g_p|^2 * |h_p|^2
 * silu is evaluated in fp32 (expf), squares accumulated in fp64. */
lrm_status lrm_score_glu(const lrm_pairs* pairs, const lrm_mat* A, const lrm_mat* B,
                         const lrm_mat* G, float* score, void* ws, size_t ws_bytes, void* stream);

/* Per-expert top-quota selection (page 1, bullets "Квоты до вычислений" and
 * "Отбор по метрике LRM"): expert e keeps M_e = min(quota[e], n_e) of its n_e
 * pairs, those with the largest score, ties broken by lower pair index.  The
 * kept pairs are then given dense packed rows, expert blocks back to back
 * with no padding and pairs ascending inside a block (bullet
 * "Физическое уплотнение"):
 *   offsets  device [E+1]: offsets[e] = M_0 + ... + M_{e-1}
 *   kept     device [N]:   kept[offsets[e] + i] = i-th kept pair of e (only
 *                          the first offsets[E] entries are written)
 *   pos      device [N]:   packed row of p, or -1 if p is dropped
 * quota: HOST [E] int32 (fixed by a controller for the call), read during the
 * call (passed with the kernel arguments for E <= 512, else copied
 * stream-ordered into ws); negative quotas are rejected (LRM_ERR_QUOTA).  With
 * LRM_QUOTA_ON_DEVICE it is a device [E] int32 array read by the kernels
 * (negative entries keep nothing).
 * flags: LRM_KEEP_ALL ignores score and quota and keeps every pair;
 * LRM_QUOTA_ON_DEVICE as above; other bits: LRM_ERR_UNSUPPORTED.
 * Under HIP graph capture, host quotas of up to 512 experts are frozen into
 * the graph at capture; host quotas of more than 512 experts would be re-read
 * by a stream copy at every replay, so such a call returns
 * LRM_ERR_UNSUPPORTED on a capturing stream (use LRM_QUOTA_ON_DEVICE).
 * ws: device scratch of lrm_select_workspace_size(pairs) bytes; its first word
 * receives device-detected index errors (see lrm_check_device_errors). */
lrm_status lrm_select(const lrm_pairs* pairs, const float* score, const int32_t* quota,
                      uint32_t flags, int32_t* pos, int32_t* offsets, int32_t* kept, void* ws,
                      size_t ws_bytes, void* stream);
size_t lrm_select_workspace_size(const lrm_pairs* pairs);

/* lrm_select for callers that cannot allocate memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * selection, results and flags, with its scratch in a device array of the
 * library, LRM_SELECT_STATIC_SCRATCH_BYTES per GPU, held from the first use
 * on a GPU until the process ends.  Calls no allocation routine.  Returns
 * LRM_ERR_WORKSPACE, having enqueued nothing, when
 * lrm_select_workspace_size(pairs) exceeds that size (for example more than
 * about a million pairs with 4096 experts).  Every call on one GPU uses that
 * GPU's one array: calls that overlap on one GPU (concurrent streams or
 * threads) race and give undefined results; calls ordered on one stream do
 * not.  The first call on a device also looks the array's address up. */
#define LRM_SELECT_STATIC_SCRATCH_BYTES (32u << 20)
lrm_status lrm_select_static(const lrm_pairs* pairs, const float* score, const int32_t* quota,
                             uint32_t flags, int32_t* pos, int32_t* offsets, int32_t* kept,
                             void* stream);

/* Physical compaction (page 1, bullet "Физическое уплотнение"): gathers the
 * kept rows into dense per-expert blocks,
 *   Xp[m] = w_p * (X row of p)   (rounded to X's dtype)
 *   Gp[m] = G row of p
 * for m < offsets[E], p = kept[m].  Either output may be NULL to skip it.
 * Xp: device [max_rows][X.cols], Gp: device [max_rows][G.cols], both of the
 * inputs' dtype and dense (ld = cols).  max_rows is the caller's capacity; it
 * must be >= offsets[E] (guaranteed by max_rows >= min(N, sum of quotas)). */
lrm_status lrm_compact(const lrm_pairs* pairs, const int32_t* kept, const int32_t* offsets,
                       int32_t max_rows, const lrm_mat* X, const lrm_mat* G, void* Xp, void* Gp,
                       void* stream);

/* Compaction into dense blocks per receiver and expert (page 1, bullets
 * "Перераспределение" and "Физическое уплотнение"): lrm_compact with packed
 * row m written to row dst[m] of Xp and Gp instead of row m.
 * dst: device [max_rows] int32, the receiver-major row of every expert-major
 * packed row, as lrm_receiver_layout writes it (receiver g's rows from
 * send_off[g], expert e's inside them from blk_off[g][e]); NULL is the
 * identity (lrm_compact).  dst must map the rows m < offsets[E] one to one
 * into [0, max_rows); a row whose dst lies outside is not written. */
lrm_status lrm_compact_rows(const lrm_pairs* pairs, const int32_t* kept, const int32_t* offsets,
                            int32_t max_rows, const int32_t* dst, const lrm_mat* X,
                            const lrm_mat* G, void* Xp, void* Gp, void* stream);

/* Variable-size grouped GEMMs on the packed blocks, no zero padding (page 1,
 * bullet "Физическое уплотнение"): for every expert e with packed rows
 * [offsets[e], offsets[e+1]) of Gp [rows][d_out] and Xp [rows][d_in]:
 *   dW[e]  = Gp_e^T Xp_e        fp32 [d_out][d_in]   (0 when M_e = 0)
 *   dXp_e  = Gp_e W_e           fp32 [M_e][d_in]     (row m of dXp)
 * W: device, expert e at W + e*w_stride elements, [d_out][d_in] row-major.
 * dtype applies to Gp, Xp, W; bf16 runs on MFMA with fp32 accumulation, fp32
 * with fp32 FMA.  dW or dXp may be NULL to skip that product (W may then be
 * NULL).  Rows of dXp at or beyond offsets[E] are not written.  d_in and d_out
 * are each 1..2^20-1 (LRM_ERR_SHAPE otherwise).
 * ws: device scratch of lrm_grouped_bwd_workspace_size(E) bytes. */
lrm_status lrm_grouped_bwd(int32_t E, const int32_t* offsets, int32_t max_rows, int32_t dtype,
                           const void* Gp, const void* Xp, const void* W, int64_t w_stride,
                           int32_t d_in, int32_t d_out, float* dW, float* dXp, void* ws,
                           size_t ws_bytes, void* stream);
size_t lrm_grouped_bwd_workspace_size(int32_t E);

/* Return to the original layout (page 1, bullet "Физическое уплотнение"):
 *   TOKEN: dX[t] = sum over the pairs p of t with pos[p] >= 0, in pair order,
 *          of w_p * dXp[pos[p]]; 0 for tokens with no kept pair
 *   PAIR:  dX[p] = w_p * dXp[pos[p]], or 0 if pos[p] < 0
 * dXp: device fp32 [*][d_in] dense; dX: device fp32 [T or N][d_in] dense.
 * ws: device scratch of lrm_unpermute_workspace_size(pairs) bytes. */
lrm_status lrm_unpermute(const lrm_pairs* pairs, const int32_t* pos, const float* dXp,
                         int32_t d_in, int32_t out_rows, float* dX, void* ws, size_t ws_bytes,
                         void* stream);
size_t lrm_unpermute_workspace_size(const lrm_pairs* pairs);

/* ------------------------------------------------------ quota controller */

/* Quotas before the computation (page 1, section "Что делает LRMoE: полный
 * прямой проход, обрезанный обратный", bullet "Квоты до вычислений"; page 2,
 * bullet "Des quotas avant le calcul"): from the number of pairs routed to
 * each expert and one budget of pairs this GPU may carry through the
 * backward pass (the memory and network limits), water-filling caps that
 * trim the most loaded experts first.  HOST function, no GPU work:
 *   tau = the largest integer with sum_e min(counts[e], tau) <= budget;
 *   quota[e] = min(counts[e], tau), plus one for the first
 *   budget - sum_e min(counts[e], tau) experts (lowest index) with
 *   counts[e] > tau; with budget >= sum counts, quota = counts.
 * So sum quota = min(budget, sum counts) and the largest quota is the
 * smallest possible for that total.
 * counts: host [E] >= 0; quota: host [E] output (may alias counts).
 * LRM_ERR_QUOTA if a count or the budget is negative. */
lrm_status lrm_quota_waterfill(int32_t E, const int32_t* counts, int64_t budget, int32_t* quota);

/* The same controller on the GPU, in stream order (same section and rule as
 * lrm_quota_waterfill; integer arithmetic, so the quotas are identical), so
 * that controller and backward run on one stream with no host round trip and
 * can be captured in one HIP graph at any E:
 *   pairs:  the routed pairs of the layer call (E is taken from it).
 *   counts: device [E] int32 pairs per expert (negative entries count as 0),
 *           or NULL: the counts are those of the pairs, computed here (pairs
 *           with an expert or token out of range are not counted, and the
 *           workspace error word reports them, see lrm_check_device_errors).
 *   budget: pairs this GPU may carry through the backward pass, >= 0 (host
 *           value, fixed for the call).
 *   quota:  device [E] int32 output, ready for LRM_QUOTA_ON_DEVICE.
 * ws: device scratch of lrm_quota_waterfill_device_workspace_size(pairs)
 * bytes.  LRM_ERR_QUOTA if budget < 0. */
lrm_status lrm_quota_waterfill_device(const lrm_pairs* pairs, const int32_t* counts,
                                      int64_t budget, int32_t* quota, void* ws, size_t ws_bytes,
                                      void* stream);
size_t lrm_quota_waterfill_device_workspace_size(const lrm_pairs* pairs);

/* ----------------------------------------- redistribution onto replicas */

/* Redistribution of the kept pairs over the copies of their expert (page 1,
 * section "Что делает LRMoE: полный прямой проход, обрезанный обратный",
 * bullet "Перераспределение"; page 2, same section, bullet
 * "Redistribution"): an integer assignment of each expert's kept pairs to
 * the GPUs holding a replica of it, minimising the peak per-GPU load; no
 * replica is created.  HOST function: it enqueues nothing and touches no
 * device memory (a controller-side step on E x G numbers).
 *   kept:    host [E], M_e >= 0 kept pairs of expert e (offsets[e+1] -
 *            offsets[e] of a selection).
 *   replica: host [E][G] uint8, nonzero where GPU g holds a copy of expert e.
 *   base:    host [G] load already on GPU g (pairs, >= 0), or NULL for zeros.
 *   cap:     host [G] most pairs GPU g may take (>= 0), or NULL for no limit.
 *   assign:  host [E][G] int32 output x[e][g] >= 0, zero where there is no
 *            replica, each row summing to kept[e].
 *   peak:    host output, max over g of base[g] + sum_e x[e][g], the minimum
 *            over all such assignments (exact).
 * Load is counted in pairs: the experts of one layer have equal shapes, so a
 * kept pair costs the same work on any replica.  The optimum is unique, the
 * assignment in general is not; this one is deterministic.
 * host_ws: host scratch of lrm_redistribute_workspace_size(E, G) bytes.
 * E in 1..4096, G in 1..1024.  LRM_ERR_INFEASIBLE if an expert with kept
 * pairs has no replica or the capacities cannot hold every kept pair (assign
 * and peak are then not written). */
lrm_status lrm_redistribute(int32_t E, int32_t G, const int32_t* kept, const uint8_t* replica,
                            const int64_t* base, const int64_t* cap, int32_t* assign,
                            int64_t* peak, void* host_ws, size_t host_ws_bytes);
size_t lrm_redistribute_workspace_size(int32_t E, int32_t G);

/* Receiver-major layout of the packed rows (page 1, bullet "Физическое
 * уплотнение": dense blocks per receiver and expert) for an assignment of
 * lrm_redistribute copied to the device:
 *   offsets:  device [E+1] of a selection (expert e's rows offsets[e] ..).
 *   assign:   device [E][G] int32 x[e][g].
 *   send_off: device [G+1] output, first row of receiver g's block.
 *   blk_off:  device [G][E+1] output, first row of expert e inside receiver
 *             g's block, relative to send_off[g] (blk_off[g][E] = its rows).
 *   dst:      device [max_rows] output, dst[m] = receiver-major row of packed
 *             row m, for m < min(offsets[E], max_rows); later rows untouched.
 * Receiver g's block holds experts 0..E-1 in order, x[e][g] rows each;
 * expert e's rows, in packed order, go to its replicas in ascending g.
 * ws: device scratch of lrm_receiver_layout_workspace_size(E, G) bytes; its
 * first word is the device error word: lrm_check_device_errors(ws) reports
 * LRM_ERR_INDEX if some x[e][g] < 0 or a row of assign does not sum to
 * offsets[e+1] - offsets[e] (dst is then unspecified). */
lrm_status lrm_receiver_layout(int32_t E, int32_t G, const int32_t* offsets,
                               const int32_t* assign, int32_t max_rows, int32_t* send_off,
                               int32_t* blk_off, int32_t* dst, void* ws, size_t ws_bytes,
                               void* stream);
size_t lrm_receiver_layout_workspace_size(int32_t E, int32_t G);

/* ------------------------------------------------------- the fused call */

typedef struct lrm_problem {
  int32_t kind;    /* lrm_kind */
  uint32_t flags;  /* LRM_KEEP_ALL, LRM_DW_BF16, LRM_QUOTA_ON_DEVICE, LRM_DEBUG_CHECKS,
                      LRM_GATHER_LOADS */
  int32_t dtype;   /* lrm_dtype of every dense input */
  int32_t _pad;
  lrm_pairs pairs;
  /* LINEAR: one projection y = W_e x per pair.  X: saved input (d_in cols,
   * TOKEN or PAIR), G: incoming gradient at the output (d_out cols, TOKEN or
   * PAIR), W: device [E][d_out][d_in] at stride w_stride, quota: HOST [E]
   * (device [E] with LRM_QUOTA_ON_DEVICE). */
  lrm_mat X;
  lrm_mat G;
  const void* W;
  int64_t w_stride;
  int32_t d_in, d_out;   /* each 1..2^20-1 */
  const int32_t* quota;
  /* SWIGLU: expert MLP W_down (silu(W_gate x) * (W_up x)).  X: saved input
   * (H cols, TOKEN), G: incoming gradient at the layer output (H cols,
   * TOKEN), A, B: saved gate/up pre-activations (I cols, PAIR), weights
   * W_gate, W_up device [E][I][H], W_down device [E][H][I] (dense, stride
   * I*H), quotas HOST [E] per projection (device [E] with
   * LRM_QUOTA_ON_DEVICE).  Host quotas are read during the call. */
  lrm_mat A;
  lrm_mat B;
  const void* W_gate;
  const void* W_up;
  const void* W_down;
  int32_t H, I;          /* each 1..2^20-1 */
  const int32_t* quota_down;
  const int32_t* quota_gate;
  const int32_t* quota_up;
  /* SWIGLU, optional (NULL = computed from A and B): device [N] fp64, the
   * squared norm |silu(a_p) * b_p|^2 of every pair's down-projection input,
   * saved by the forward pass.  The down score then reads this one number per
   * pair instead of the rows of A and B; compaction and the SwiGLU backward
   * still read A and B, for the kept rows only.  8-byte aligned. */
  const double* h_sumsq;
} lrm_problem;

typedef struct lrm_outputs {
  /* dW pointers: fp32, or bf16 storage with LRM_DW_BF16 */
  float* dW;      /* LINEAR: device [E][d_out][d_in] */
  float* dW_gate; /* SWIGLU: device [E][I][H] */
  float* dW_up;   /* SWIGLU: device [E][I][H] */
  float* dW_down; /* SWIGLU: device [E][H][I] */
  float* dX;      /* device fp32, rows of X's layout (T or N) x d_in (or H) */
  /* Optional (NULL = not returned).  LINEAR / SwiGLU down stage: */
  float* score;     /* device [N] */
  int32_t* pos;     /* device [N] */
  int32_t* offsets; /* device [E+1] */
  /* SwiGLU gate/up stages, indexed by the down stage's packed row m: */
  float* score_gate;       /* device [max down rows] */
  float* score_up;         /* device [max down rows] */
  int32_t* pos_gate;       /* device [max down rows]: gate packed row or -1 */
  int32_t* pos_up;         /* device [max down rows] */
  int32_t* offsets_gate;   /* device [E+1] */
  int32_t* offsets_up;     /* device [E+1] */
  /* SwiGLU: the unscaled hidden gradient u = W_down^T g of every down-kept
   * row, fp32 [max down rows][I] (the input of the gate/up scores). */
  float* dH;
} lrm_outputs;

/* The whole pruned expert backward of one layer call (the page "LRMoE
 * урезает обратный проход MoE ...", section "Что делает LRMoE: полный прямой
 * проход, обрезанный обратный": quotas fixed before the backward, bullet
 * "Квоты до вычислений"; scoring and selection, bullet "Отбор по метрике
 * LRM"; packing, variable-size GEMMs and the return to the original layout,
 * bullet "Физическое уплотнение"; the SwiGLU order down -> gate/up is the
 * reading stated at the top of this header), all steps enqueued on one
 * stream with no device->host synchronisation:
 *   LINEAR: score -> select -> compact -> grouped GEMM (dW, dXp) -> unpermute.
 *   SWIGLU: down score -> select -> compact (g, w*h) -> grouped GEMM
 *           (dW_down, u = W_down^T g) -> SwiGLU backward ga = u*b*silu'(a),
 *           gb = u*silu(a) with gate/up scores -> gate and up select among
 *           the down-kept pairs -> compact -> grouped GEMMs (dW_gate, dW_up,
 *           dX rows) -> unpermute.
 * With LRM_KEEP_ALL every pair is kept and no score or select runs (the
 * unpruned baseline on the same kernels).  With LRM_DEBUG_CHECKS the call
 * synchronises its stream at the end and returns LRM_ERR_INDEX when a kernel
 * found an index error (the only flag that makes the call synchronous).
 * "max down rows" is min(N, sum of quota_down), or N with LRM_KEEP_ALL; with
 * LRM_QUOTA_ON_DEVICE the caller, which knows its quotas, sizes those outputs
 * by the same rule (only rows of kept pairs are written).
 * HIP graph capture: a captured call freezes the packed sizes the host
 * computed from the quotas at capture, and host quotas of up to 512 experts
 * (passed by value).  Host quotas of more than 512 experts are copied by a
 * stream copy that a replay would repeat from the host array, so the call
 * returns LRM_ERR_UNSUPPORTED on a capturing stream; device quotas
 * (LRM_QUOTA_ON_DEVICE) are read at every replay and sized for every pair.
 * Should a selection ever keep more rows than its packed buffers hold, the
 * later experts keep fewer, every access stays inside the workspace and the
 * outputs, and lrm_check_device_errors reports LRM_ERR_WORKSPACE.
 * ws: device scratch of lrm_workspace_size(prob) bytes, 256-byte aligned. */
lrm_status lrm_expert_backward(const lrm_problem* prob, const lrm_outputs* out, void* ws,
                               size_t ws_bytes, void* stream);

/* lrm_expert_backward, additionally recording events[i] (a hipEvent_t created
 * by the caller, passed as void*) on the stream at boundary i, for each
 * i < n_events with events[i] != NULL.  Every grouped-GEMM launch sits
 * between two boundaries of its own:
 *   LINEAR: 0 start, 1 after score, 2 after select, 3 after compaction,
 *           4 after the dW launch, 5 after the dX launch, 6 after unpermute
 *           (end).  fp32 runs both products in one launch: 4 and 5 are its end.
 *   SWIGLU: 0 start, 1 after the down score, 2 after the down select, 3 after
 *           the down compaction, 4 after the down dW launch, 5 after the down
 *           dX launch (u), 6 after the SwiGLU backward with the gate/up
 *           scores, 7 after the gate/up selects, 8 after the gate/up
 *           compaction, 9 after the gate dW launch, 10 after the gate dX
 *           launch, 11 after the up dW launch, 12 after the up dX launch,
 *           13 after unpermute (end).  When the gate/up selections keep every
 *           down-kept row, one launch computes both input-gradient products
 *           (between 9 and 10) and 12 coincides with 11; with bf16 inputs,
 *           I a multiple of 64 and no LRM_GATHER_LOADS, one launch also
 *           computes both weight gradients (between 8 and 9), the
 *           input-gradient launch sits between 9 and 10, and 11 and 12
 *           coincide with 10.
 * The time between consecutive events is that stage's device time on the
 * stream (for profiling; the results are those of lrm_expert_backward). */
lrm_status lrm_expert_backward_events(const lrm_problem* prob, const lrm_outputs* out, void* ws,
                                      size_t ws_bytes, void* stream, void* const* events,
                                      int32_t n_events);

/* Workspace bytes lrm_expert_backward needs for prob (0 if prob is invalid).
 * Packed buffers are sized from the host quotas: min(N, sum of quotas) rows. */
size_t lrm_workspace_size(const lrm_problem* prob);

/* Upper bound on the kept rows of a selection with these host quotas:
 * min(N, sum of quota[e]); -1 if a quota is negative or an argument is NULL. */
int64_t lrm_max_kept(int32_t N, int32_t E, const int32_t* quota);

/* Synchronises the stream, then reads the device error word at the start of
 * a workspace used by lrm_select, lrm_expert_backward or lrm_receiver_layout:
 * LRM_OK, or LRM_ERR_INDEX if an expert index was out of range or token[]
 * was out of range or decreasing (such pairs are treated as absent), or a
 * replica assignment did not match the kept counts; otherwise
 * LRM_ERR_WORKSPACE if a selection kept more rows than the packed buffers of
 * the call were sized for (a captured call replayed with other quotas); and
 * clears it. */
lrm_status lrm_check_device_errors(void* ws, void* stream);

/* Static description of a status code. */
const char* lrm_status_string(lrm_status s);

/* Library version (major*10000 + minor*100 + patch). */
int32_t lrm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LRM_H_ */

/*
 * rma.h -- C ABI of librma.so: Top-K+phi residual-mass-accounting decode on
 * AMD MI355X (gfx950).
 *
 * Method: "Residual-Mass Accounting for Partial-KV Decoding" (arXiv
 * 2604.05438).  §1 summarises it: at prefill, fixed-size positive-feature
 * summaries (S, u) are built over the non-anchor mid-region of each kv head;
 * at decode, exact unnormalised terms are computed over the sink/tail anchors
 * and the retrieved tokens, the retrieved tokens' feature contributions are
 * subtracted from the summaries, the residual numerator/denominator estimate
 * phi(q)^T S_res, phi(q)^T u_res is added in the unnormalised domain, and a
 * single normalisation follows (§4.3, Eq. 10).  The KV cache format is left
 * unchanged (the v1 abstract: the module keeps backbone weights and the
 * KV-cache format unchanged), so every call reads the caller's cache in place.
 *
 * Conventions shared by every call
 *  - All pointers are DEVICE pointers unless stated otherwise.  The caller owns
 *    every buffer, including the workspace.  The library never allocates or
 *    frees memory and never synchronises: each call validates its arguments on
 *    the host, then enqueues kernels on `stream` (a hipStream_t; NULL = the
 *    null stream) and returns.  Device-side faults surface at the caller's
 *    next synchronisation.
 *  - A "unit" is one (request, layer, kv head).  Units are numbered
 *    u = 0..n_units-1; parameter set p = u % n_param_sets serves unit u.
 *  - KV cache view (rma_kv): element (u, t, j) of K (or V) lives at
 *    k[u*unit_stride + t*d + j], rows t = 0..t_cap-1, d = head dim.  K and V
 *    share dtype, strides and shape.  Positions [0, L) are the prefill
 *    segment; [L, L + n_gen) are generated tokens.
 *  - Span (rma_span): anchors A = [0, n_sink) u [L - n_tail, L), mid-region
 *    M = [n_sink, L - n_tail) of size L_mid = L - n_sink - n_tail (page §3,
 *    Eq. 2), generated tokens [L, L + n_gen) (exact, never in the residual,
 *    page §3 before Eq. 5 and Eq. 11).
 *  - Query q: fp32 [n_units][G][d]; query head g of unit u is the g-th of the G
 *    query heads that share the kv head (GQA).
 *  - Supported now: d in {64, 128}; m in {64, 128}; G in 1..8; K/V dtype
 *    RMA_F32 or RMA_BF16; phi_k storage RMA_F32 or RMA_BF16.  Anything else
 *    returns RMA_ERR_UNSUPPORTED.
 *  - Alignment: every device pointer must be 16-byte aligned, and unit_stride
 *    a multiple of 8 elements; otherwise RMA_ERR_INVALID_ARG.
 *  - Errors: validation happens before anything is enqueued; on an error
 *    nothing is launched and the outputs are untouched.  rma_last_error()
 *    gives a message for the calling thread's last failed call.
 *  - Workspace: calls that need scratch take (workspace, workspace_bytes);
 *    rma_workspace_bytes() gives the size.  A workspace holds per-call scratch
 *    only: every byte a call's kernels read from it is written earlier in the
 *    same call, so it needs no initialisation and one workspace can serve any
 *    sequence of calls on one stream.  Calls that may run concurrently need
 *    distinct workspaces.
 *  - NaN/Inf inputs are not checked; outputs are then unspecified (no fault).
 */
#ifndef RMA_H_
#define RMA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RMA_ABI_VERSION 9

/* Most events one kernel trace can hold (rma_trace_arm). */
#define RMA_TRACE_MAX_EVENTS 16

typedef enum {
  RMA_OK = 0,
  RMA_ERR_INVALID_ARG = -1,  /* null pointer, bad size, misalignment, K > L_mid, ... */
  RMA_ERR_UNSUPPORTED = -2,  /* d, m, G or dtype outside the supported set */
  RMA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required */
  RMA_ERR_HIP = -4           /* a kernel launch failed */
} rma_status;

typedef enum { RMA_F32 = 0, RMA_BF16 = 1 } rma_dtype;

/* Read-only view of one KV cache (K and V of n_units units). */
typedef struct {
  const void* k;
  const void* v;
  int32_t dtype;        /* rma_dtype of K and V */
  int32_t n_units;
  int64_t t_cap;        /* rows per unit */
  int64_t unit_stride;  /* elements between consecutive units (>= t_cap*d) */
  int32_t d;            /* head dim (d_h = d_v) */
  int32_t reserved;
} rma_kv;

/* Prefill segment and generated tokens, identical for every unit. */
typedef struct {
  int64_t L;            /* prefill length */
  int32_t n_sink;
  int32_t n_tail;
  int64_t n_gen;        /* generated tokens visible to this decode step */
} rma_span;

/* Operation ids for rma_workspace_bytes(). */
#define RMA_OP_BUILD_SUMMARIES 1
#define RMA_OP_DECODE_TOPK 2
#define RMA_OP_DECODE_MERGE 3
#define RMA_OP_DECODE_FULL 4
#define RMA_OP_DECODE 5

/* rma_build_summaries_range() flags. */
#define RMA_BUILD_ACCUMULATE 1u    /* add to S, u (and raise kappa) instead of overwriting */

/* rma_decode_merge() flags (page §5.2 Table 1 and §7.1 Table 3 variants). */
#define RMA_MERGE_SUB 0u           /* Top-K+phi: subtract retrieved tokens (default) */
#define RMA_MERGE_NO_RESIDUAL 1u   /* selection-only Top-K: drop the residual */
#define RMA_MERGE_NO_SUBTRACT 2u   /* NoSub: add the whole-mid estimate, no subtraction */

/* Weights of n_param_sets MLP feature maps (rma_phi_mlp_features), device
 * pointers.  The matrices are bf16 in the matrix-core tile order: a matrix W
 * with N outputs and K inputs (element W[n][k]) is stored per parameter set as
 * [K/32][N/16][64][8], element (n, k) at
 *   ((k/32 * N/16 + n/16) * 64 + (n%16 + 16 * (k%32)/8)) * 8 + k%8,
 * so that the weight pieces one wave multiplies together are one contiguous
 * kilobyte.  Biases and the ReZero scalars are fp32.  Width RMA_PHI_MLP_WIDTH. */
#define RMA_PHI_MLP_WIDTH 512
typedef struct {
  const uint16_t* W_in;   /* bf16, N = 512, K = d, tile order */
  const float* b_in;      /* fp32 [n_param_sets][512] */
  const uint16_t* W_1;    /* bf16, N = K = 512, tile order */
  const float* b_1;       /* fp32 [n_param_sets][512] */
  const uint16_t* W_2;    /* bf16, N = K = 512, tile order */
  const float* b_2;       /* fp32 [n_param_sets][512] */
  const float* alpha;     /* fp32 [n_param_sets]: the ReZero block scale */
  const uint16_t* W_o;    /* bf16, N = m, K = 512, tile order */
  const float* b_o;       /* fp32 [n_param_sets][m] */
} rma_phi_mlp;

/*
 * rma_phi_mlp_features -- the pages' feature-map family (§4.4: head-specific
 * one-block ReZero MLPs; App. C.1 "Why positivity matters": exponentiated
 * outputs; §8 "Scope and runtime": d_phi = 64, with parameter totals that fix
 * width 512 and biases on every layer; the block's activation is not given,
 * ReLU here):
 *     h0 = W_in x + b_in,   h1 = h0 + alpha (W_2 relu(W_1 h0 + b_1) + b_2),
 *     phi[u][r][:] = exp(W_o h1 + b_o),    parameter set p = u % n_param_sets.
 * The products run on the matrix cores with bf16 operands (x, h0, relu(.), h1
 * are rounded to bf16, nearest even, before they enter a product) and fp32
 * sums; biases, alpha, the residual sum and exp are fp32.
 * x:   [n_units][rows][d] of x_dtype, unit stride x_unit_stride elements, row
 *      stride d.  For the keys of the mid-region pass k + n_sink*d, rows =
 *      L_mid and the cache's unit stride (one map per kv head); for decode
 *      queries [U][G][d] pass n_units = U*G, rows = 1 (one map per query head).
 * phi: [n_units][rows][m] of phi_dtype, dense (m = 64 or 128).
 * Stored phi_k rows feed rma_build_summaries with Wk == NULL; phi_q rows feed
 * rma_decode_merge as phi_q.
 * Errors: RMA_ERR_INVALID_ARG (NULL pointers, sizes, alignment),
 * RMA_ERR_UNSUPPORTED (d, m or dtypes).
 */
rma_status rma_phi_mlp_features(const void* x, int32_t x_dtype, int32_t n_units, int64_t rows,
                                int64_t x_unit_stride, int32_t d, const rma_phi_mlp* weights,
                                int32_t m, int32_t n_param_sets, void* phi, int32_t phi_dtype,
                                void* stream);

/*
 * rma_phi_features -- positive feature map (page App. C.1 "Why positivity
 * matters"; the elu+1 form of the workloads):
 *     phi[u][r][:] = elu(W[p] x[u][r] + b[p]) + 1,   p = u % n_param_sets.
 * x:   [n_units][rows][d] of x_dtype, unit stride x_unit_stride elements, row
 *      stride d.
 * W:   fp32 [n_param_sets][m][d] row-major;  b: fp32 [n_param_sets][m].
 * phi: [n_units][rows][m] of phi_dtype, dense.
 * Used at decode for f = phi_q(q) (rows = G).  Arithmetic is fp32.
 */
rma_status rma_phi_features(const void* x, int32_t x_dtype, int32_t n_units, int64_t rows,
                            int64_t x_unit_stride, int32_t d, const float* W, const float* b,
                            int32_t m, int32_t n_param_sets, void* phi, int32_t phi_dtype,
                            void* stream);

/*
 * rma_build_summaries -- prefill summaries over the mid-region (page §1 and
 * §4.1; Eq. 6):
 *     Phi_K[u][i][:] = phi_k(k[u][n_sink + i]),  i = 0..L_mid-1
 *     S[u]   = sum_i Phi_K[u][i] v[u][n_sink+i]^T     fp32 [m][d]
 *     u_[u]  = sum_i Phi_K[u][i]                       fp32 [m]
 *     kappa[u] >= max_i ||k[u][n_sink+i]||_2           fp32 (an upper bound)
 * If Wk != NULL, phi_k rows are computed (elu(Wk[p] k + bk[p]) + 1), rounded
 * to phi_dtype and written to phi_k; S and u are formed from the rounded rows
 * so that the rows later subtracted at decode are exactly those summed here.
 * With Wk != NULL, bf16 keys/values and phi_dtype RMA_BF16, phi_k may be NULL:
 * the rows are then not stored, and rma_decode_merge recomputes the retrieved
 * ones bit for bit from their keys (the same projection and rounding).
 * If Wk == NULL (bk ignored), phi_k is an INPUT holding the rows (any positive
 * features, e.g. for an ideal-factorisation check) and is only read.
 * phi_k: NULL or [n_units][L_mid][m] of phi_dtype, dense.  S, u_, kappa
 * overwritten.
 * Needs L_mid >= 0 (L_mid == 0 gives S = u = 0, kappa = 0).
 * Workspace: rma_workspace_bytes(RMA_OP_BUILD_SUMMARIES, ...).
 */
rma_status rma_build_summaries(const rma_kv* kv, const rma_span* span, const float* Wk,
                               const float* bk, int32_t m, int32_t n_param_sets, void* phi_k,
                               int32_t phi_dtype, float* S, float* u_, float* kappa,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * rma_build_summaries_range -- the same summaries over the mid-region positions
 * [m_begin, m_end) only (tokens n_sink + m_begin .. n_sink + m_end - 1), for a
 * prefill that arrives in pieces or a shared prefix whose summaries are reused.
 * The summaries are plain sums over tokens (page §4.1, Eq. 6), so they add over
 * disjoint token sets: pieces appended with RMA_BUILD_ACCUMULATE give the
 * whole-range result up to fp32 summation order (kappa exactly: a maximum).
 * flags 0: S, u_, kappa are overwritten with the range's sums;
 * flags RMA_BUILD_ACCUMULATE: S += range sums, u_ += range sums,
 *   kappa = max(kappa, range bound); S, u_, kappa must hold earlier results.
 * phi_k rows m_begin .. m_end-1 of [n_units][L_mid][m] are written (or read,
 * with Wk == NULL); the rest of phi_k is untouched.  Other arguments as for
 * rma_build_summaries, which equals this call on [0, L_mid) with flags 0.
 * Errors: RMA_ERR_INVALID_ARG for 0 <= m_begin <= m_end <= L_mid violated or
 * unknown flags.  Workspace: rma_workspace_bytes(RMA_OP_BUILD_SUMMARIES, ...)
 * for the same span suffices for any range.
 */
rma_status rma_build_summaries_range(const rma_kv* kv, const rma_span* span, int64_t m_begin,
                                     int64_t m_end, uint32_t flags, const float* Wk,
                                     const float* bk, int32_t m, int32_t n_param_sets,
                                     void* phi_k, int32_t phi_dtype, float* S, float* u_,
                                     float* kappa, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * rma_decode_topk -- exhaustive Top-K over the mid-region (page §1: exhaustive
 * Top-K is the control selector that fixes the exact support; §3 Eq. 3: K(q)
 * is a subset of M of size K).  For every query head it ranks all mid tokens
 * by the exact real value of q.k_i (scaling by 1/sqrt(d) does not change the
 * order), ties to the lower position, and returns the K winners.
 * q:       fp32 [n_units][G][d].
 * kappa:   fp32 [n_units], from rma_build_summaries (bounds the fp32 scoring
 *          error; selection is exact for any inputs).
 * idx:     int32 [n_units][G][K]: absolute positions in [n_sink, L - n_tail),
 *          ascending.
 * sel_scores: fp32 [n_units][G][K]: s_i = fl32(q.k_i) / sqrt(d) of idx[...],
 *          consumed by rma_decode_merge.
 * 0 <= K <= L_mid.  K == 0 writes nothing.
 * Workspace: rma_workspace_bytes(RMA_OP_DECODE_TOPK, ...) (depends on G, K).
 */
rma_status rma_decode_topk(const float* q, int32_t G, const rma_kv* kv, const rma_span* span,
                           const float* kappa, int32_t K, int32_t* idx, float* sel_scores,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * rma_decode_merge -- exact branch, retrieved-token subtraction, residual
 * estimate and single normalisation (page §3 Eq. 3-4 and 11, §4.2 Eq. 9,
 * §4.3 Eq. 10):
 *   E = A u K(q) u Gen, s_i = q.k_i/sqrt(d), m* = max_{i in E} s_i,
 *   N_E = sum_E e^{s_i - m*} v_i,  Z_E = sum_E e^{s_i - m*},
 *   w_i = f.Phi_K[i] (i in K(q)),  f = phi_q[u][g],
 *   nu_R = S^T f - sum_{K(q)} w_i v_i,  Z_R = max(u^T f - sum_{K(q)} w_i, 0)
 *   (both exactly 0 when K == L_mid; the clamp is the page's App. C.1 guard
 *   against subtraction artifacts),
 *   y = (N_E + e^{-m*} nu_R) / (Z_E + e^{-m*} Z_R).
 * q: fp32 [n_units][G][d];  phi_q: fp32 [n_units][G][m] (any positive
 * features; rma_phi_features gives phi_q), or NULL with Wq, bq given: then
 * f = elu(Wq q + bq) + 1 is computed inside this call (fp32; Wq fp32
 * [n_param_sets][m][d], bq fp32 [n_param_sets][m], unit u uses set
 * u % n_param_sets), which spares the separate rma_phi_features launch.  Wq,
 * bq are ignored when phi_q is given.  idx, sel_scores as written by
 * rma_decode_topk (K per head).  phi_k, S, u_ as written/used by
 * rma_build_summaries.  When the subtraction needs Phi_K rows (RMA_MERGE_SUB,
 * 0 < K < L_mid) and phi_k is NULL, they are recomputed from the retrieved
 * keys with Wk, bk (fp32 [n_param_sets][m][d], [n_param_sets][m]; unit u uses
 * set u % n_param_sets) exactly as rma_build_summaries computed the summed
 * rows: bf16 keys and phi_dtype RMA_BF16 only (else RMA_ERR_UNSUPPORTED).
 * Wk, bk are ignored when phi_k is given.
 * flags: RMA_MERGE_SUB, RMA_MERGE_NO_RESIDUAL (selection-only Top-K) or
 *        RMA_MERGE_NO_SUBTRACT (NoSub).
 * y: fp32 [n_units][G][d].  stats: NULL or fp32 [n_units][G][4] =
 *    (m*, Z_E, Z_R (unshifted, after the clamp), sum_{K(q)} w_i); the last
 *    is 0 unless the subtraction runs (RMA_MERGE_SUB with 0 < K < L_mid).
 * With K == L_mid (RMA_MERGE_SUB) the residual is exactly zero: no phi_k row
 * is read, and phi_k, Wk and bk may all be NULL.
 * Requires n_sink + n_tail + n_gen + K > 0.
 * Workspace: rma_workspace_bytes(RMA_OP_DECODE_MERGE, ...).
 */
rma_status rma_decode_merge(const float* q, const float* phi_q, const float* Wq,
                            const float* bq, int32_t G, const rma_kv* kv,
                            const rma_span* span, const int32_t* idx, const float* sel_scores,
                            int32_t K, const void* phi_k, int32_t phi_dtype, const float* Wk,
                            const float* bk, int32_t n_param_sets, int32_t m, const float* S,
                            const float* u_, uint32_t flags, float* y, float* stats,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * rma_decode -- one decode step of Top-K+phi: rma_decode_topk followed by
 * rma_decode_merge in one call (page §1: the exhaustive Top-K fixes the exact
 * support; §3 Eq. 3-4 and 11, §4.2 Eq. 9, §4.3 Eq. 10: exact terms, the
 * subtraction, the residual and one normalisation).  The scan of
 * rma_decode_topk runs first; then one block per query head selects its K
 * tokens and merges them in the same kernel, the selection going straight
 * from on-chip memory into the gathers (when the head's candidate lists and
 * selection fit the block's on-chip memory and the phi_k rows are stored;
 * otherwise the separate select and merge kernels run on the same scan).
 * Results equal the two calls' up to fp32 summation order: the same indices
 * and selected scores, y within a few fp32 ulps.
 * Arguments as for those two calls: q, G, kv, span, kappa, K as for
 * rma_decode_topk; phi_q, Wq, bq, phi_k, phi_dtype, Wk, bk, n_param_sets, m,
 * S, u_, flags, y, stats as for rma_decode_merge.  idx, sel_scores: NULL (not
 * written) or, both given, [n_units][G][K] outputs as rma_decode_topk writes
 * them.  kappa may be NULL when K == 0.
 * Workspace: rma_workspace_bytes(RMA_OP_DECODE, ...) (depends on G, K, m).
 * Errors: those of the two calls; RMA_ERR_INVALID_ARG also when only one of
 * idx and sel_scores is given.
 */
rma_status rma_decode(const float* q, const float* phi_q, const float* Wq, const float* bq, int32_t G,
                      const rma_kv* kv, const rma_span* span, const float* kappa, int32_t K,
                      const void* phi_k, int32_t phi_dtype, const float* Wk, const float* bk,
                      int32_t n_param_sets, int32_t m, const float* S, const float* u_,
                      uint32_t flags, int32_t* idx, float* sel_scores, float* y, float* stats,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * rma_decode_full -- full exact attention of every query head over its unit's
 * whole context, the reference the method approximates (page §3 Eq. 1, with
 * the generated tokens of Eq. 11), and the page's comparison diagnostics
 * (§6: entropy of the attention restricted to the mid-region; §7.1 Table 3:
 * relative l1 output error and the residual log-partition error, for which
 * log Z_R over R(q) = M minus K(q) is given here):
 *   s_i = q.k_i / sqrt(d),  i in [0, L + n_gen),
 *   y_full = sum_i e^{s_i} v_i / sum_i e^{s_i}.
 * q: fp32 [n_units][G][d].  idx: NULL, or [n_units][G][K] ascending positions
 *    inside M (as written by rma_decode_topk) that form K(q); entries outside M
 *    or out of order make diag[2] meaningless but cannot fault.  K == 0 means
 *    R(q) = M.  y_cmp: NULL, or fp32 [n_units][G][d], an output to compare with
 *    y_full (e.g. rma_decode_merge's y).
 * y_full: fp32 [n_units][G][d].  diag: NULL or fp32 [n_units][G][8] =
 *    (log Z_full, log Z_mid, log Z_R, H_mid, rel_l1, max s_i, 0, 0), natural
 *    logs of the unshifted sums sum e^{s_i} over the whole context, over M and
 *    over R(q) (NaN when idx is NULL and K > 0; -inf for an empty set),
 *    H_mid = -sum_M p_i log p_i / log L_mid with p renormalised over M (NaN
 *    when L_mid < 2), rel_l1 = sum_j |y_cmp - y_full| / sum_j |y_full| (NaN
 *    without y_cmp).
 * K and V are read once per unit for all G heads; fp32 arithmetic.
 * Workspace: rma_workspace_bytes(RMA_OP_DECODE_FULL, ...) (depends on G).
 */
rma_status rma_decode_full(const float* q, int32_t G, const rma_kv* kv, const rma_span* span,
                           const int32_t* idx, int32_t K, const float* y_cmp, float* y_full,
                           float* diag, void* workspace, size_t workspace_bytes, void* stream);

/*
 * rma_decode_topk_static -- rma_decode_topk with no workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The call's scratch
 * lives in a device array the library owns, RMA_STATIC_SCRATCH_BYTES on every
 * GPU the library runs on (held until the process ends); the call itself
 * allocates and frees nothing.  Arguments, results and errors are those of
 * rma_decode_topk, plus RMA_ERR_WORKSPACE (before anything is enqueued) when
 * the call needs more scratch than the array holds, i.e. when
 * rma_workspace_bytes(RMA_OP_DECODE_TOPK, ...) exceeds RMA_STATIC_SCRATCH_BYTES
 * (the 1B and 3B single-layer workloads at 32K and 64K fit), and RMA_ERR_HIP
 * when the array's address cannot be obtained on the current device.  Every
 * call on one GPU uses that GPU's one array: calls that may overlap on one GPU
 * (other streams, other threads) race, and the caller must serialise them.
 * Nothing in the array needs to start at zero: every byte a call reads from it
 * is written earlier in the same call.
 */
#define RMA_STATIC_SCRATCH_BYTES (16u << 20)
rma_status rma_decode_topk_static(const float* q, int32_t G, const rma_kv* kv, const rma_span* span,
                                  const float* kappa, int32_t K, int32_t* idx, float* sel_scores,
                                  void* stream);

/* Workspace bytes for `op` (one of RMA_OP_*), at least 256; 0 on invalid
 * arguments.  G and K are ignored for RMA_OP_BUILD_SUMMARIES; m is ignored for
 * RMA_OP_DECODE_TOPK and RMA_OP_DECODE_FULL; K is ignored for
 * RMA_OP_DECODE_FULL. */
size_t rma_workspace_bytes(int32_t op, const rma_kv* kv, const rma_span* span, int32_t G,
                           int32_t K, int32_t m);

/* Static text for a status code; never NULL. */
const char* rma_status_string(int32_t status);

/* Message for the calling thread's last failed call ("" if none). */
const char* rma_last_error(void);

/* RMA_ABI_VERSION of the loaded library. */
int32_t rma_abi_version(void);

/* Per-kernel timing, for benchmarks and profiling only (not part of the
 * method).  Arms a trace for the next entry point called on this thread that
 * enqueues kernels: its j-th kernel (j = 0 .. n_events/2 - 1; later kernels are
 * not timed) is launched through hipExtLaunchKernel with events[2j] and
 * events[2j+1], which its dispatch stamps when the kernel starts and when it
 * ends, so their elapsed time is the kernel's execution time alone.  The call
 * then disarms the trace.  `events` are hipEvent_t handles owned by the
 * caller, created with timing enabled on the stream's device; the library
 * keeps the handles until that call and never frees them.  n_events == 0
 * disarms.  Thread-local state; do not arm a trace for a call that is being
 * captured into a graph.
 * Errors: RMA_ERR_INVALID_ARG (n_events not 0 and not even in 2..16, NULL
 * handle). */
rma_status rma_trace_arm(void* const* events, int32_t n_events);

/* Kernels timed by the last traced call on this thread. */
int32_t rma_trace_count(void);

/* Name of the j-th timed kernel of that call (0-based), or NULL. */
const char* rma_trace_name(int32_t j);

/* Streaming-read ceiling, for benchmarks only (not part of the method): reads
 * the device range [p, p + bytes) once with `blocks` workgroups of 256 threads,
 * block b taking the b-th of `blocks` contiguous pieces, with the load form of
 * the Top-K scan (nontemporal 16-byte loads, two batches of eight per thread in
 * flight), and writes to sink[b] the XOR of the 32-bit words of block b's
 * piece (the XOR of all `blocks` words is that of the whole range).  Its time
 * is what the device allows for reading those bytes with that grid: the
 * reference the scan's own rate is compared with.  p (device, 16-byte aligned,
 * `bytes` a positive multiple of 16) and sink (device, `blocks` uint32,
 * overwritten) belong to the caller.  Enqueues one kernel on `stream` (a trace
 * armed by rma_trace_arm times it); never synchronizes.
 * Errors: RMA_ERR_INVALID_ARG (NULL pointer, misalignment, bytes not a
 * positive multiple of 16, blocks outside 1..2^20); RMA_ERR_HIP. */
rma_status rma_stream_read(const void* p, int64_t bytes, int32_t blocks, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RMA_H_ */

/*
 * pisa.h -- C ABI of libpisa, block-sparse attention with training-free block
 * selection for AMD Instinct MI355X (gfx950).
 *
 * The operation is the forward pass the following pages describe together:
 *   [PISA]  "PISA: Piecewise Sparse Attention Is Wiser for Efficient Diffusion
 *           Transformers" -- technical summary, section 2 (core algorithm:
 *           o_t = N_t / D_t with exact terms over the selected blocks and a
 *           block-level Taylor term around the mean key for every other
 *           block, inside both N_t and D_t; hardware implementation:
 *           precompute centroids and value sums, then one fused
 *           online-softmax kernel).
 *   [PIVOT] "PIVOT slashes sparse-attention indexer cost 4x ..." -- section
 *           "Two observations behind PIVOT", steps 1-4 (one averaged proxy
 *           query per group of g consecutive queries scores the blocks; the
 *           proxy's candidate list is re-ranked per member).
 *   [SWA]   "Sliding Window Attention" -- causal window 0 <= t - s < w
 *           (section "How the window widens with depth"); window-aware kernels
 *           skip blocks outside the kept set entirely (related term
 *           "FlashAttention").
 *
 * Three calls make one forward pass, all asynchronous on the caller's stream:
 *   pisa_block_stats     mean-pooled block statistics (stage A)
 *   pisa_indexer_topk    block scores and top-k selection (stage B)
 *   pisa_sparse_attn_fwd exact attention over kept blocks + per-block
 *                        first-order Taylor tail for the rest (stage C)
 *
 * Conventions shared by every call
 *   Layout   Q: [B, Hq, L, d]; K, V: [B, Hkv, L, d]; O like Q.  Contiguous,
 *            d fastest, base pointers 16-byte aligned.  Query head h uses KV
 *            head h * Hkv / Hq (consecutive query heads share a KV head).
 *   Blocks   bs = block; n_blk = ceil(L / bs); block j holds tokens
 *            [j*bs, min(L, (j+1)*bs)) and n_j of them.
 *   Memory   The caller allocates and owns every buffer (inputs, statistics,
 *            index lists, outputs, workspace).  The library allocates no
 *            device memory and keeps no global state other than a
 *            thread-local error text and the fixed decode scratch of
 *            pisa_decode_fwd_noalloc (a static device array); every other
 *            call is re-entrant.
 *   Errors   Every precondition is checked on the host before anything is
 *            launched.  On failure a call returns a non-zero status, writes
 *            nothing and launches nothing; pisa_last_error() gives the
 *            reason.  A failed launch returns PISA_E_HIP.
 *   Async    Calls only enqueue kernels on `stream`; no host synchronisation
 *            and no host<->device copies happen inside.
 *   Results  Deterministic: bitwise identical from run to run.
 *   Inputs   Q, K, V values must be finite.
 */
#ifndef PISA_H
#define PISA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PISA_ABI_VERSION 2

typedef enum {
  PISA_OK = 0,
  PISA_E_ARG = 1,          /* invalid argument (null, shape, range, alignment) */
  PISA_E_UNSUPPORTED = 2,  /* valid but not implemented (d, block size, ...) */
  PISA_E_WORKSPACE = 3,    /* workspace missing or too small */
  PISA_E_HIP = 4           /* a HIP launch failed; see pisa_last_error() */
} pisa_status;

typedef enum { PISA_BF16 = 0, PISA_F32 = 1 } pisa_dtype;

/* Treatment of non-kept candidate blocks ([PISA] section 2). */
typedef enum {
  PISA_TAYLOR_NONE = 0,    /* drop them (keep-or-drop block sparsity) */
  PISA_TAYLOR_ORDER0 = 1,  /* exp(q.kbar_j) * sum_n v_n ; exp(q.kbar_j) * n_j */
  PISA_TAYLOR_ORDER1 = 2,  /* adds exp(q.kbar_j) * q H_j to the numerator */
  PISA_TAYLOR_HYBRID = 3   /* zero order per block, plus one global first-order
                              term q Hbar * sum_j exp(q.kbar_j) in the numerator,
                              Hbar = mean of H_j over all blocks of the (b, kv
                              head) ([PISA] section 2, hybrid order); on a
                              causal row the mean over the blocks it may see as
                              Taylor candidates, [0, lo_r), so that no later
                              token enters the row */
} pisa_taylor;

/* Problem statement.  Supported today: d in {64, 128}; block in {64, 128};
 * Hq / Hkv in {1, 2, 4, 8}; n_blk <= 1024; topk + sink <= 256;
 * n_cand <= 256. */
typedef struct {
  int32_t B, Hq, Hkv, L, d;
  int32_t dtype;    /* pisa_dtype of Q, K, V and O */
  int32_t block;    /* bs: key and query block size in tokens */
  int32_t topk;     /* k kept blocks per row beyond the window / own block; 0 allowed */
  int32_t window;   /* causal window w in tokens (0 = none); requires causal */
  int32_t group;    /* 0: one selection row per query block (mean-pooled query);
                       g >= 1: one selection row per token, PIVOT proxies of g
                       consecutive queries (block % g == 0); g = 1 with
                       n_cand >= n_blk is the dense per-token indexer */
  int32_t n_cand;   /* PIVOT proxy list length C >= topk (C == topk: PIVOT-Reuse) */
  int32_t causal;   /* 0 or 1 */
  int32_t taylor;   /* pisa_taylor */
  float scale;      /* softmax scale; <= 0 selects 1/sqrt(d) */
  int32_t sink;     /* attention sinks ([SWA] glossary): the first min(sink,
                       |cand_r|) candidate blocks of every row are always kept
                       exactly and head its kept list; the top-k is chosen
                       among the other candidates.  topk + sink <= 256. */
  float route_lambda; /* covariance-aware routing ([PISA] section 2): >= 0;
                       when > 0 every selection score (block rows, PIVOT
                       proxies and members) is the attention score plus
                       route_lambda * mcov_j.  Needs taylor != NONE.  Defined
                       for non-causal rows only: the page measures the norm
                       against the mean over all blocks of bidirectional
                       attention, which on a causal row would carry later
                       tokens; causal with route_lambda > 0 returns
                       PISA_E_UNSUPPORTED. */
} pisa_params;

/* Block statistics ([PISA] precompute; [PIVOT] step 2).  Caller-allocated,
 * sizes from pisa_stats_layout().
 *   qsel  dtype [B, Hq, n_sel, d]: RNE_dtype(float64 mean of the query rows of
 *         block i) for group == 0 (n_sel = n_blk), or of the g queries of
 *         PIVOT group gamma (n_sel = ceil(L / g); a last partial group
 *         averages its actual members)
 *   ksel  dtype [B, Hkv, n_blk, d]: RNE_dtype(float64 mean key of block j)
 *   kbar  fp32 [B, Hkv, n_blk, d]: the mean key, rounded to fp32 (Taylor term)
 *   vsum  fp32 [B, Hkv, n_blk, d]: sum of the block's value rows
 *   HT    bf16 for bf16 inputs and fp32 for fp32 inputs.  ORDER1:
 *         [B, Hkv, n_blk, d, d], the transposed first-order matrix,
 *         HT[e][c] = sum_n v_{n,e} (k_{n,c} - kbar_c).  HYBRID, non-causal:
 *         [B, Hkv, d, d], the transposed mean of those matrices over the n_blk
 *         blocks of the (b, kv head).  HYBRID, causal: [B, Hkv, n_blk, d, d],
 *         entry lo the transposed mean over blocks [0, lo) (entry 0 is zero),
 *         the matrix of every row whose Taylor candidates are [0, lo).  Not
 *         used by the other modes.
 *   mcov  fp32 [B, Hkv, n_blk]: ||H_j - Hbar||_F, the covariance norm of block
 *         j against the mean first-order matrix ([PISA] covariance-aware
 *         routing; the pages' norm read as Frobenius), written and read when
 *         route_lambda > 0
 * kbar and vsum are read only when taylor != NONE, HT only for ORDER1 and
 * HYBRID, mcov only with routing; they may be NULL otherwise. */
typedef struct {
  void *qsel;
  void *ksel;
  float *kbar;
  float *vsum;
  void *HT;
  float *mcov;
} pisa_stats;

/* ---- host-only queries (no GPU needed) ---------------------------------- */

/* Check a problem statement; PISA_OK if every call can run it. */
pisa_status pisa_validate(const pisa_params *p);

/* Byte sizes of the six statistics buffers, in pisa_stats field order
 * (qsel, ksel, kbar, vsum, HT, mcov); 0 for a buffer the problem does not use. */
pisa_status pisa_stats_layout(const pisa_params *p, size_t bytes[6]);

/* Byte sizes of the index list idx (int32 [B, Hq, n_rows, topk + sink],
 * n_rows = n_blk for group == 0 else L) and of the PIVOT proxy list cand
 * (int32 [B, Hq, ceil(L / g), n_cand]; 0 when group == 0). */
pisa_status pisa_index_layout(const pisa_params *p, size_t bytes[2]);

/* Workspace bytes call `op` needs (0 = block_stats, 1 = indexer_topk,
 * 2 = sparse_attn_fwd, 3 = decode_fwd).  decode_fwd always needs one
 * (fp32 split-K partials).  block_stats needs one for the HYBRID order with bf16
 * inputs and for routing (fp32 partial sums of the mean first-order matrix and
 * an fp32 copy of it).  sparse_attn_fwd needs one for PIVOT rows in bf16 with
 * taylor NONE when the rows' kept sets fit the key-gathered kernel (at most
 * 1024 blocks, its LDS budget): K and V^T of every 64-key unit in MFMA
 * fragment order, 4 * B * Hkv * n_blk * block * d bytes; 0 otherwise.  Workspaces are 16-byte aligned;
 * their contents need not be initialised and are garbage afterwards.  Every
 * other call and mode needs none.  A non-NULL workspace of at least
 * PISA_DIAG_BYTES passed to pisa_indexer_topk receives diagnostic counters
 * (int32: rows selected, rows whose fast selection was not certified and went
 * to a float64 re-score or an exact comparison, rows or candidates decided by
 * exact comparison).  The counters are updated with atomics on one address
 * and slow the call down; they are for diagnosis, not for timed runs. */
#define PISA_DIAG_BYTES 64
pisa_status pisa_workspace_size(const pisa_params *p, int op, size_t *bytes);

/* ---- the hot path ------------------------------------------------------- */

/* Stage A.  Reads Q, K, V; writes every non-NULL statistics buffer of *out
 * (qsel and ksel are required; kbar and vsum when taylor != NONE, HT for
 * ORDER1 and HYBRID, mcov with routing).  ws: at least
 * pisa_workspace_size(p, 0) bytes, else PISA_E_WORKSPACE. */
pisa_status pisa_block_stats(const pisa_params *p, const void *Q, const void *K,
                             const void *V, const pisa_stats *out, void *ws,
                             size_t ws_bytes, hipStream_t stream);

/* Stage B ([PISA] routing by attention score, covariance-aware with
 * route_lambda > 0; [PIVOT] steps 1-4; [SWA] window).  Per selection row r
 * the score of candidate block j is the exact real dot product
 * qsel_r . ksel_j (PIVOT members: q_t . ksel_j), plus route_lambda * mcov_j
 * (the product and sum exact, mcov as given in the statistics);
 * the kept set T_r is the top-min(k, |cand_r|) candidates, ties to the lower
 * block index.  Candidates: every block when non-causal; when causal, blocks
 * [0, lo_r) where lo_r = blk(max(0, start_r - w + 1)) (w > 0) or the row's
 * own block (w = 0), start_r being the first token of the row; the range
 * [lo_r, own block] is kept implicitly and not stored.  With sinks, the
 * first c0 = min(sink, |cand_r|) candidates are kept and listed first, and
 * the top-k is taken over the candidates from c0 on.  PIVOT: the proxy of
 * group gamma keeps the top-min(C, |cand| - c0) of its first member's
 * candidates past their sinks; each member keeps its own sinks and the
 * top-min(k, C') of that list by its own score.
 * Writes idx (ascending, -1 padded to topk + sink) and, if non-NULL, cand. */
pisa_status pisa_indexer_topk(const pisa_params *p, const void *Q, const pisa_stats *stats,
                              int32_t *idx, int32_t *cand, void *ws, size_t ws_bytes,
                              hipStream_t stream);

/* Stage C ([PISA] section 2 with the per-block first-order term).  For token
 * t in selection row r, with q_s = scale * q_t:
 *   E_t = tokens of the blocks in T_r u [lo_r, own] (s <= t when causal)
 *   U_t = candidates of r not in T_r (empty when taylor == NONE)
 *   N_t = sum_{s in E_t} e^{q_s.k_s} v_s
 *       + sum_{j in U_t} e^{q_s.kbar_j} (vsum_j + [ORDER1] q_s H_j)
 *       + [HYBRID] (q_s Hbar) sum_{j in U_t} e^{q_s.kbar_j}
 *   D_t = sum_{s in E_t} e^{q_s.k_s} + sum_{j in U_t} e^{q_s.kbar_j} n_j
 *   O_t = N_t / D_t rounded to nearest-even in dtype;
 *   lse_t = max-shifted ln D_t (fp32 [B, Hq, L]) if lse != NULL.
 * idx may come from pisa_indexer_topk or from the caller (e.g. lists reused
 * from another layer, [HyLRA] section 2.3).  T_r is the set of the row's
 * entries j with 0 <= j < |cand_r|; every other entry (the -1 padding, a
 * block of the window range [lo_r, own] or past it, any other value) is
 * dropped on the device, so no entry reads outside Q, K, V or the statistics.
 * Block rows (group == 0) accept the entries in any order and repeated.
 * PIVOT rows (group >= 1) need the kept entries in ascending order (repeats
 * and dropped entries may sit anywhere); pisa_indexer_topk writes them so.
 * ws: at least pisa_workspace_size(p, 2) bytes, else PISA_E_WORKSPACE. */
pisa_status pisa_sparse_attn_fwd(const pisa_params *p, const void *Q, const void *K,
                                 const void *V, const pisa_stats *stats, const int32_t *idx,
                                 void *O, float *lse, void *ws, size_t ws_bytes,
                                 hipStream_t stream);

/* ---- decode: one new token per (b, query head) ---------------------------
 * [HyLRA] section 2.3 (hybrid inference: sensitive layers select the top-k
 * blocks and pass them on, tolerant layers reuse an earlier layer's lists
 * and attend to that part of the cache only); [SWA] the w-slot ring buffer.
 * The token at position pos (0 <= pos < L) is the causal token row t = pos
 * of the prefill path: p must be causal; L is the capacity of the cache,
 * whose keys 0 .. pos are valid; group and n_cand are not used.
 *   q      dtype [B, Hq, d]
 *   K, V   dtype [B, Hkv, L, d], the cache (ring == 0), or
 *          dtype [B, Hkv, ring, d], a ring buffer with token i in slot i mod ring
 *   stats  block statistics of the cache (pisa_block_stats over it); only
 *          statistics of blocks before the row's window range are read (for
 *          HYBRID the entry lo of HT, the mean over [0, lo)), so cache slots
 *          after pos may hold anything finite: qsel is not used
 *   idx    int32 [B, Hq, topk + sink] kept lists (any order, repeats allowed);
 *          entries outside the candidates [0, lo) are ignored
 *   O      dtype [B, Hq, d];  lse  fp32 [B, Hq] or NULL
 * pisa_decode_topk writes the lists of a sensitive layer: the sinks, then
 * the top-min(k, |cand| - c0) of candidates [c0, lo) by q . ksel_j
 * (+ route_lambda * mcov_j), certified exactly as pisa_indexer_topk.
 * pisa_decode_fwd: exact terms over the listed blocks and the window range
 * [lo, own] (keys s <= pos), Taylor terms (taylor mode of p) over the other
 * candidates.  ring > 0: a pure sliding window over the last `ring` tokens
 * (max(0, pos - ring + 1) .. pos exactly); needs topk == 0, sink == 0,
 * taylor == NONE and window == ring; idx and stats are not read.
 * ws: at least pisa_workspace_size(p, 3) bytes (split-K partials). */
pisa_status pisa_decode_topk(const pisa_params *p, int32_t pos, const void *q, const pisa_stats *stats,
                             int32_t *idx, hipStream_t stream);
pisa_status pisa_decode_fwd(const pisa_params *p, int32_t pos, int32_t ring, const void *q,
                            const void *K, const void *V, const pisa_stats *stats,
                            const int32_t *idx, void *O, float *lse, void *ws, size_t ws_bytes,
                            hipStream_t stream);

/* ---- decode without a workspace -------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * operation, arguments, results and error behaviour as pisa_decode_fwd, with
 * the split-K partials in a fixed scratch array of the library instead of a
 * caller workspace.  The array holds PISA_DECODE_SCRATCH_BYTES; a problem
 * whose pisa_workspace_size(p, 3) exceeds it returns PISA_E_WORKSPACE before
 * anything is launched.  Each device the library runs on holds its own copy
 * until the process ends.  Nothing is allocated: no hipMalloc / hipFree and no
 * allocating library call.  Every call on a device shares that device's
 * array, so calls that overlap on one device (other streams, other threads)
 * race; calls in stream order do not.  Stale contents from an earlier call do
 * not matter: every partial is written before it is read. */
#define PISA_DECODE_SCRATCH_BYTES ((size_t)16 << 20)
pisa_status pisa_decode_fwd_noalloc(const pisa_params *p, int32_t pos, int32_t ring, const void *q,
                                    const void *K, const void *V, const pisa_stats *stats,
                                    const int32_t *idx, void *O, float *lse, hipStream_t stream);

/* ---- errors and version -------------------------------------------------- */
const char *pisa_status_string(pisa_status s);
const char *pisa_last_error(void);  /* thread-local detail of the last failure */
int pisa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PISA_H */

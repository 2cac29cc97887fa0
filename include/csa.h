/*
 * csa.h -- C ABI of the MI355X (gfx950) compressed-sparse-attention (CSA) forward path.
 *
 * The path has four calls, run in this order on one HIP stream:
 *   csa_indexer_score      Lightning-Indexer scores with the compressed causal mask
 *   csa_topk               per-row top-k with global ids
 *   csa_sparse_attn_fwd    sliding-window + top-k attention with a per-head sink;
 *                          also emits lse, the sink+window log-mass and the head-summed
 *                          compressed probabilities (cmass) the teacher needs
 *   csa_indexer_teacher_kl paper-equivalent teacher, KL(teacher || indexer softmax)
 *                          and the loss reduction
 * and, after it, csa_indexer_loss_bwd (the loss gradients for the indexer inputs).
 * Two calls merge steps: csa_indexer_topk (scores + top-k without the score matrix) and
 * csa_sparse_attn_kl_fwd (attention + teacher + KL + loss for the sparse loss).
 *
 * Sources cited below by tag:
 *  [I5776]  page "[Bug] DSV4 unfused CSA indexer loss uses a compressed-only teacher
 *           instead of the full CSA attention distribution" (Megatron-LM issue 5776),
 *           its Megatron-LM code excerpts (csa.py, dsa.py, dsa_kernels.py) and its
 *           discussion thread (proposal comment, review comment).
 *  [PR8539] page "Megatron-LM pull request 8539" (cuDNN frontend 1.26 defaults):
 *           item 1 (global top-k ids), item 2 (bottom-right causal offsets).
 *
 * Conventions shared by every call
 *  - Every tensor pointer is DEVICE memory allocated and owned by the caller (the
 *    library allocates nothing, frees nothing and keeps no pointer after a call
 *    returns).  Tensors are dense row-major; the shapes below are in elements.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only enqueues
 *    kernels on it and returns: no host synchronisation, no device->host copy.
 *  - Misuse that the host can see (null pointers, sizes out of range, an unsupported
 *    shape or dtype) is rejected BEFORE anything is enqueued, with CSA_ERR_INVALID or
 *    CSA_ERR_UNSUPPORTED; a launch failure returns CSA_ERR_HIP.  csa_last_error()
 *    then returns a message (thread-local, valid until the next call on the thread).
 *  - Device-side data is a precondition and is not validated (that would need a sync):
 *    cu_seqlens_q/k non-decreasing, starting at 0 and ending at total_q / total_k;
 *    ids either -1 or a valid global key row.
 *  - A packed (THD) batch of num_seqs segments is described by csa_layout_t; a BSHD
 *    batch of b sequences of length S is the special case cu_seqlens_q = [0,S,..,bS]
 *    (one code path for both).
 *  - Row geometry (per query row t of segment s), used by every call:
 *      r = t - cu_q[s],  i = r + 1 + off[s]  (1-based absolute position),
 *      S_k(s) = cu_k[s+1] - cu_k[s],
 *      n_valid(t) = clamp(floor(i / compress_ratio), 0, S_k(s))
 *    i.e. query position i sees compressed keys j < i // ratio ([I5776], csa.py SBHD
 *    causal-mask excerpt), aligned bottom-right per segment ([PR8539], item 2).
 *  - k_eff = min(topk, max_seqlen_k) ([I5776], csa.py excerpts: k = min(index_topk,
 *    n_compressed) for SBHD, min(index_topk, max_seqlen_compressed) for THD).
 */
#ifndef CSA_H_
#define CSA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA_OK = 0,
  CSA_ERR_INVALID = 1,      /* bad argument visible on the host */
  CSA_ERR_UNSUPPORTED = 2,  /* valid request without a kernel (shape / dtype) */
  CSA_ERR_HIP = 3           /* a HIP launch failed */
} csa_status_t;

typedef enum { CSA_F32 = 0, CSA_BF16 = 1 } csa_dtype_t;

typedef struct {
  int32_t num_seqs;          /* B >= 1: sequences (BSHD) or documents (THD) */
  int32_t total_q;           /* T >= 0: query rows (rows of q, kv, q_idx, weights) */
  int32_t total_k;           /* T_k >= 1: compressed key rows (rows of ckv, k_idx) */
  int32_t max_seqlen_q;      /* host copy of max_s (cu_q[s+1]-cu_q[s]), >= 1 */
  int32_t max_seqlen_k;      /* host copy of max_s S_k(s), >= 1 */
  int32_t compress_ratio;    /* >= 1 */
  const int32_t *cu_seqlens_q;     /* device [B+1] */
  const int32_t *cu_seqlens_k;     /* device [B+1]: compressed-key row boundaries
                                      ([I5776] THD excerpt: cumsum(seg_len_q // ratio)) */
  const int32_t *q_causal_offsets; /* device [B] per-segment offsets, or NULL for the
                                      bottom-right default S_k(s)*ratio - seg_len_q(s)
                                      ([PR8539], item 2).  A query chunk scored against
                                      its key prefix passes off = chunk start. */
  const int32_t *cu_seqlens_q_unpadded; /* device [B+1] or NULL (no padding).  Real segment
                                      boundaries of a batch padded to a static shape: row t
                                      of segment s is a padding row iff
                                      t - cu_q[s] >= cu_unp[s+1] - cu_unp[s] (a trailing
                                      dummy segment has real length 0).  The forward calls
                                      compute padding rows like any other row; the loss
                                      leaves them out (teacher 0, kl_row 0, no gradient)
                                      while the mean-mode divisor stays the physical
                                      total_q ([I5776] fused-path excerpt, step 4b; review
                                      comment on the padded-THD divisor).  Precondition:
                                      0 <= real length <= physical length per segment. */
} csa_layout_t;

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *csa_last_error(void);

/* k_eff = min(topk, L->max_seqlen_k), the width of ids/cmass; -1 if L or topk is bad. */
int32_t csa_k_eff(const csa_layout_t *L, int32_t topk);

/*
 * csa_indexer_score -- Lightning-Indexer scores.
 *   scores[t, j] = sum_h ws[t,h] * max(0, q_idx[t,h,:] . k_idx[cu_k[s]+j, :])  j < n_valid(t)
 *   scores[t, j] = -inf                                    n_valid(t) <= j < max_seqlen_k
 * with ws[t,h] = fp32(weights[t,h] * idx_scale) rounded to fp32 ([I5776], csa.py SBHD
 * excerpt: weights.float() * indexer.softmax_scale).  The ReLU/weighted-head-sum form
 * is the Lightning-Indexer score; the pages only show the scale folding and the
 * per-indexer-head intermediate [Sq, B, H_index, Sk], which this call never stores.
 * One k_idx row is shared by every indexer head.
 *   q_idx   [T, Hi, Di]  dtype dt        k_idx [T_k, Di] dtype dt
 *   weights [T, Hi] fp32                 scores [T, ld_scores] fp32, ld_scores >= max_seqlen_k;
 *                                        columns >= max_seqlen_k are not written.
 * Supported: dt = CSA_BF16 with Di in {32, 64, 128}; dt = CSA_F32 with Di in {32, 64, 128};
 * 1 <= Hi <= 128.  Arithmetic: exact products, fp32 accumulation (MFMA), fp32 epilogue.
 */
csa_status_t csa_indexer_score(const csa_layout_t *L, const void *q_idx, const void *k_idx,
                               const float *weights, csa_dtype_t dt, int32_t Hi, int32_t Di,
                               float idx_scale, float *scores, int64_t ld_scores, void *stream);

/*
 * csa_topk -- per-row top-k selection.
 *   K_t = min(k_eff, n_valid(t)) columns j < n_valid(t) with the largest scores[t, j];
 *   ties go to the lower j.  ids[t, 0..K_t) = cu_k[s] + j in ascending order (global
 *   ids: [PR8539] item 1, b*S_k + local for BSHD; flat packed ids for THD), and
 *   ids[t, K_t..k_eff) = -1 ([I5776], csa.py sparse-attention excerpt: picks beyond the
 *   causal limit become -1).  Only columns j < n_valid(t) are read.
 *   scores [T, ld_scores] fp32 (finite or -inf; no NaN);  ids [T, k_eff] int32;
 *   sel_scores [T, k_eff] fp32 or NULL: slot j receives the score of ids[t, j] (-inf at -1
 *       slots), so that csa_indexer_teacher_kl / csa_indexer_loss_bwd can read the selected
 *       scores in place (scores_selected = 1) instead of gathering them from the rows.
 * Supported: max_seqlen_k <= 16384, 1 <= topk.
 */
csa_status_t csa_topk(const csa_layout_t *L, const float *scores, int64_t ld_scores,
                      int32_t topk, int32_t *ids, float *sel_scores, void *stream);

/*
 * csa_indexer_topk -- csa_indexer_score and csa_topk in one pass that never stores the
 * [T, max_seqlen_k] score matrix (the per-indexer-head and per-row score tensors are the
 * memory cost the pages point at: [I5776] review comment on the unfused path).  Each
 * 16-token block's score rows are built in on-chip memory and selected there.
 *   ids [T, k_eff] int32: exactly csa_topk's ids of csa_indexer_score's scores (same
 *       arithmetic, same lowest-index tie rule), k_eff = min(topk, max_seqlen_k);
 *   sel_scores [T, k_eff] fp32: scores[t, ids[t,j] - cu_k[s]] at every valid slot, -inf
 *       at -1 slots -- what the sparse-loss predictor reads (pass it to
 *       csa_indexer_teacher_kl / csa_indexer_loss_bwd with scores_selected = 1);
 *   row_lse [T] fp32 or NULL: log sum_{j < n_valid(t)} exp(scores[t, j]) (-inf when
 *       n_valid(t) = 0), the dense-mode predictor's normaliser.
 * Inputs as csa_indexer_score.  Supported: dt = CSA_BF16, max_seqlen_k <= 2048 (512 for
 * Di = 128), and (Hi, Di) in
 *   {(8, 64), (16, 64), (4, 128), (8, 128)} (two 16-token blocks per workgroup): the q
 *       rows of both blocks plus 16 score rows of 64 * (ceil(max_seqlen_k / 64) + 1)
 *       floats within the 160 KiB of LDS of a compute unit (for (16, 64):
 *       max_seqlen_k <= 1024);
 *   {(32, 64), (64, 64), (16, 128), (32, 128)} (one block per workgroup, the heads taken
 *       in groups of 2 KiB of q row): 16 score rows of 64 * ceil(max_seqlen_k / 64) + 4
 *       floats within the LDS (max_seqlen_k <= 1856 for (32, 64), <= 1792 for (64, 64));
 * other shapes return CSA_ERR_UNSUPPORTED (use the two calls).
 */
csa_status_t csa_indexer_topk(const csa_layout_t *L, const void *q_idx, const void *k_idx,
                              const float *weights, csa_dtype_t dt, int32_t Hi, int32_t Di,
                              float idx_scale, int32_t topk, int32_t *ids, float *sel_scores,
                              float *row_lse, void *stream);

/*
 * csa_sparse_attn_fwd -- sliding-window + top-k compressed attention with a sink.
 * For query row t of segment s and head h ([I5776] "Paper reference", Z_h equation;
 * csa.py sparse-attention excerpt: window ids concatenated with the top-k ids, the
 * sink passed as fp32, softmax_scale on the q.k products):
 *   window rows   Wset(t) = { t' : max(cu_q[s], t - window + 1) <= t' <= t }
 *                 (the window ids are not defined on the pages; this reading takes the
 *                 `window` most recent rows of the segment, the query row included)
 *   w_ht' = scale * q[t,h,:] . kv[t',:],  c_hj = scale * q[t,h,:] . ckv[ids[t,j],:]
 *   Z_h = exp(sink[h]) + sum_W exp(w) + sum_{j: ids[t,j] >= 0} exp(c)
 *   out[t,h,:] = (sum_W exp(w) kv[t',:] + sum_j exp(c) ckv[ids[t,j],:]) / Z_h
 * One KV row per position is both key and value and is shared by every head; the sink
 * is a raw logit that carries no value.  Also written:
 *   lse[t,h]    = log Z_h
 *   lse_nc[t,h] = u_h = log(exp(sink[h]) + sum_W exp(w))   ([I5776] proposal comment)
 *   cmass[t,j]  = sum_h exp(c_hj - lse[t,h]) for ids[t,j] >= 0, else 0
 *   q [T, H, D], kv [T, D], ckv [T_k, D]: dtype dt;   out [T, H, D]: dtype dt
 *   sink [H] fp32;  ids [T, k_eff] int32;  lse, lse_nc [T, H] fp32;
 *   cmass [T, k_eff] fp32 or NULL (then not computed).
 * softmax_scale must be finite and > 0 (CSA_ERR_INVALID otherwise).
 * Supported: dt = CSA_BF16 with D in {64, 128, 192, 256, 512}, dt = CSA_F32 with
 * D in {64, 128}; 1 <= H <= 128; 0 <= window; 0 <= k_eff <= 4096.
 * A row with no key at all and sink = -inf gets out = 0, lse = lse_nc = -inf.
 */
csa_status_t csa_sparse_attn_fwd(const csa_layout_t *L, const void *q, const void *kv,
                                 const void *ckv, const float *sink, const int32_t *ids,
                                 int32_t k_eff, int32_t window, csa_dtype_t dt, int32_t H,
                                 int32_t D, float softmax_scale, void *out, float *lse,
                                 float *lse_nc, float *cmass, void *stream);

/*
 * csa_indexer_teacher_kl -- paper-equivalent teacher, KL and loss.
 * Support C_t: sparse_loss != 0: the valid top-k slots of ids[t, :];
 *              sparse_loss == 0: every causally visible key j < n_valid(t)
 *              ([I5776] proposal comment: top-k intersected with the causally valid
 *              entries for the sparse loss, all causally visible entries for the dense).
 * Teacher ([I5776] "Paper reference", t_j equation; proposal comment, l_h and p_hj):
 *   l_h = log(exp(lse_nc[t,h]) + sum_{j in C} exp(c_hj)),  m_j = sum_h exp(c_hj - l_h),
 *   teacher_j = m_j / max(sum_{j in C} m_j, 1e-10)
 *   sparse: m_j = cmass[t, j] (the attention's own l_h);  dense: c_hj = softmax_scale *
 *   q[t,h,:] . ckv[cu_k[s]+j,:] recomputed here for every j < n_valid(t).
 * Predictor p = softmax of scores[t, .] over C (sparse: the scores at the local columns
 * ids - cu_k[s]; dense: columns 0..n_valid(t)-1) ([I5776], dsa_kernels.py excerpt).
 * scores_selected != 0 (sparse mode only): `scores` is [T, ld_scores >= k_eff], slot j
 * holding the score of ids[t, j] (sel_scores of csa_indexer_topk).
 *   kl_row[t] = sum_{j in C} teacher_j * (log(teacher_j + 1e-10) - log(p_j + 1e-10))
 *   ([I5776], dsa.py excerpt; review comment "KL numerical contract"); 0 if n_valid(t)=0.
 *   loss[0] = sum_t kl_row[t] / total_q  (every physical row is in the divisor), or the
 *   plain sum if per_token_loss != 0.  The reduction is deterministic (no atomics).
 * Arguments:
 *   scores [T, ld_scores] fp32 (from csa_indexer_score);  ids [T, k_eff] int32;
 *   sparse: cmass [T, k_eff] fp32 (q, ckv, lse_nc may be NULL);
 *   dense:  q [T, H, D], ckv [T_k, D] (dtype dt), lse_nc [T, H] fp32 (cmass may be NULL);
 *   teacher: NULL, or [T, ld_teacher] fp32 receiving the teacher (sparse: slot j at
 *            column j, 0 at -1 slots, ld_teacher >= k_eff; dense: column j < n_valid,
 *            0 beyond, ld_teacher >= max_seqlen_k);
 *   kl_row [T] fp32;  loss [1] fp32.
 * Supported (dense): dt = CSA_BF16 with D in {64, 128, 192, 256, 512}, 1 <= H <= 128,
 * max_seqlen_k <= 8192 (any dtype in sparse mode, where q and ckv are not read).
 */
csa_status_t csa_indexer_teacher_kl(const csa_layout_t *L, int32_t sparse_loss,
                                    const float *scores, int64_t ld_scores,
                                    int32_t scores_selected, const int32_t *ids, int32_t k_eff, const float *cmass,
                                    const void *q, const void *ckv, const float *lse_nc,
                                    csa_dtype_t dt, int32_t H, int32_t D, float softmax_scale,
                                    int32_t per_token_loss, float *teacher, int64_t ld_teacher,
                                    float *kl_row, float *loss, void *stream);

/*
 * csa_sparse_attn_kl_fwd -- csa_sparse_attn_fwd followed by csa_indexer_teacher_kl with
 * the sparse loss, as one call: the attention produces the per-head compressed
 * probabilities, and the teacher and the KL reduce them in the same pass ([I5776]
 * "Paper reference", t_j equation: the teacher is the attention's own head-summed
 * distribution over the compressed set, Z_h keeping the sink and window terms).
 * Computes exactly what the two calls compute, with the same arguments:
 *   out, lse, lse_nc, cmass      as csa_sparse_attn_fwd (cmass is required here);
 *   teacher, kl_row, loss        as csa_indexer_teacher_kl with sparse_loss = 1 (the
 *                                support is the valid top-k slots of ids[t, :]).
 * scores [T, ld_scores] fp32: with scores_selected != 0 slot j of row t holds the score
 * of ids[t, j] (sel_scores of csa_indexer_topk, ld_scores >= k_eff); otherwise the full
 * score rows of csa_indexer_score (ld_scores >= max_seqlen_k).
 * With scores_selected != 0 and a shape of the one-wave-per-query attention kernel
 * (dt = CSA_BF16, H <= 16, D in {64, 128}, window >= 1, k_eff <= 256) the attention
 * kernel finishes each row's teacher and KL in its epilogue and one more kernel reduces
 * the loss; every other supported shape runs the attention and teacher kernels in turn.
 * loss may be NULL: then only kl_row is written and csa_loss_reduce finishes the loss.
 * Supported: as csa_sparse_attn_fwd, with 1 <= k_eff.
 */
csa_status_t csa_sparse_attn_kl_fwd(const csa_layout_t *L, const void *q, const void *kv,
                                    const void *ckv, const float *sink, const int32_t *ids,
                                    int32_t k_eff, int32_t window, csa_dtype_t dt, int32_t H,
                                    int32_t D, float softmax_scale, const float *scores,
                                    int64_t ld_scores, int32_t scores_selected,
                                    int32_t per_token_loss, void *out, float *lse, float *lse_nc,
                                    float *cmass, float *teacher, int64_t ld_teacher,
                                    float *kl_row, float *loss, void *stream);

/*
 * csa_loss_reduce -- loss[0] = sum_t kl_row[t] / total_q, or the plain sum if
 * per_token_loss != 0 (the divisor counts every physical row: [I5776] review comment),
 * 0 for total_q = 0.  The last step of csa_indexer_teacher_kl as a call of its own, for
 * csa_sparse_attn_kl_fwd with loss = NULL.  Deterministic: one workgroup adds the rows in
 * a fixed order in fp64.  kl_row [total_q] fp32 (may be NULL if total_q = 0); loss [1].
 */
csa_status_t csa_loss_reduce(const float *kl_row, int32_t total_q, int32_t per_token_loss,
                             float *loss, void *stream);

/*
 * csa_indexer_loss_bwd -- gradients of the indexer loss for the indexer q, weights and k.
 * The step after the forward path ([I5776] proposal comment and review comment: the loss
 * keeps a custom backward that recomputes what it needs from saved tensors and returns
 * gradients only for the indexer q, weights and k; every teacher-side input is detached;
 * [PR8539] item 1: the sparse path's ids are global).  The teacher (from
 * csa_indexer_teacher_kl's `teacher` output) and the selection are inputs held fixed.
 * With the support C_t, predictor p = softmax(scores[t, C_t]) and teacher t_j of the
 * forward, and c = grad_loss / total_q (or grad_loss if per_token_loss != 0):
 *   r_j = t_j p_j / (p_j + 1e-10),  g_tj = c * (p_j * sum_{j' in C} r_j' - r_j)  (j in C),
 *   g_tj = 0 elsewhere  -- the derivative of the KL of csa_indexer_teacher_kl;
 *   with d_thj = q_idx[t,h,:] . k_idx[cu_k[s]+j,:], a = [d > 0], ws = fp32(w[t,h]*idx_scale):
 *   dq_idx[t,h,:]      = ws * sum_j g_tj a_thj k_idx[cu_k[s]+j,:]
 *   dweights[t,h]      = idx_scale * sum_j g_tj max(d_thj, 0)
 *   dk_idx[cu_k[s]+j,:] = sum_{t in s} sum_h g_tj ws a_thj q_idx[t,h,:]
 * Arguments:
 *   q_idx [T, Hi, Di], k_idx [T_k, Di] (dtype dt);  weights [T, Hi] fp32;
 *   scores [T, ld_scores] fp32 (the forward's; sparse mode with scores_selected != 0:
 *   [T, ld_scores >= k_eff] slot-aligned with ids, as csa_indexer_topk writes them);
 *   sparse: ids [T, k_eff] int32 and
 *   teacher [T, ld_teacher >= k_eff] (slot-aligned with ids); dense: ids may be NULL and
 *   teacher [T, ld_teacher >= max_seqlen_k] (column j for j < n_valid);
 *   grad_scores: workspace [T, ld_grad >= max_seqlen_k] fp32, overwritten with g;
 *   dq_idx [T, Hi, Di], dweights [T, Hi], dk_idx [T_k, Di]: fp32, overwritten (every
 *   element, including rows and keys that get no gradient).  Deterministic: no atomics.
 *   workspace: device scratch of workspace_bytes >= csa_indexer_loss_bwd_workspace(L,
 *   Hi, Di) bytes (may be NULL when that is 0), caller-owned, contents undefined after
 *   the call; it holds per-chunk partial sums of dk_idx, which a last kernel adds in a
 *   fixed order.  A smaller workspace is CSA_ERR_INVALID.
 * Supported: dt = CSA_BF16; Di in {64, 128} with Hi in {4, 8, 16, 32, 64}; sparse
 * k_eff <= 4096, dense max_seqlen_k <= 4096.
 */
csa_status_t csa_indexer_loss_bwd(const csa_layout_t *L, int32_t sparse_loss,
                                  const void *q_idx, const void *k_idx, const float *weights,
                                  csa_dtype_t dt, int32_t Hi, int32_t Di, float idx_scale,
                                  const float *scores, int64_t ld_scores, int32_t scores_selected,
                                  const int32_t *ids,
                                  int32_t k_eff, const float *teacher, int64_t ld_teacher,
                                  float grad_loss, int32_t per_token_loss, float *grad_scores,
                                  int64_t ld_grad, float *dq_idx, float *dweights, float *dk_idx,
                                  void *workspace, int64_t workspace_bytes, void *stream);

/*
 * csa_indexer_loss_bwd_noalloc -- csa_indexer_loss_bwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same gradients from the same arguments, with no grad_scores and no
 * workspace argument.  The score-gradient matrix and the dk chunk partials live in a
 * static device array of the library, CSA_NOALLOC_SCRATCH_BYTES (128 MiB) per GPU, held
 * by each GPU the library runs on until the process ends; its device address is looked up
 * on the first call on each device (with that device current).  The call allocates and
 * frees nothing.  Outputs dq_idx, dweights, dk_idx are caller-owned as in
 * csa_indexer_loss_bwd and equal its outputs bit for bit.
 * Scratch needed: total_q * ld * 4 bytes (ld = max_seqlen_k rounded up to 64) rounded up to
 * 256, plus csa_indexer_loss_bwd_workspace(L, Hi, Di); a layout needing more than
 * CSA_NOALLOC_SCRATCH_BYTES is CSA_ERR_INVALID before anything is enqueued (use
 * csa_indexer_loss_bwd with caller workspaces then).
 * Every call on one GPU uses that GPU's one array and leaves its contents behind: calls
 * that overlap on one GPU (two streams, two threads) race and must be serialised by the
 * caller.  Nothing in the array has to start at a particular value.
 */
#define CSA_NOALLOC_SCRATCH_BYTES (128ll << 20)
csa_status_t csa_indexer_loss_bwd_noalloc(const csa_layout_t *L, int32_t sparse_loss,
                                          const void *q_idx, const void *k_idx, const float *weights,
                                          csa_dtype_t dt, int32_t Hi, int32_t Di, float idx_scale,
                                          const float *scores, int64_t ld_scores, int32_t scores_selected,
                                          const int32_t *ids, int32_t k_eff, const float *teacher,
                                          int64_t ld_teacher, float grad_loss, int32_t per_token_loss,
                                          float *dq_idx, float *dweights, float *dk_idx, void *stream);

/* Bytes of device workspace csa_indexer_loss_bwd needs for this layout and indexer
 * shape (0: none); -1 for an invalid layout or an unsupported shape (message in
 * csa_last_error).  Host-only: reads nothing on the device. */
int64_t csa_indexer_loss_bwd_workspace(const csa_layout_t *L, int32_t Hi, int32_t Di);

/*
 * csa_cp_plan -- host-only layout of one rank's share of context-parallel (CP) scoring.
 * ([PR8539], item 2 and its test plan: the CP scorers score each query chunk against its
 * document's key prefix, cropped at the chunk end, and pass the chunk's absolute causal
 * offset explicitly, so every row sees exactly its absolute causal keys whatever the
 * default alignment.)
 * Each of num_docs documents (doc_len[d] query rows, packed back to back; doc_len[d] /
 * ratio compressed keys, packed back to back) is cut into 2*cp_size chunks of
 * doc_len[d] / (2*cp_size) rows; rank cp_rank holds chunks cp_rank and
 * 2*cp_size-1-cp_rank of every document (the zig-zag split that evens out causal work).
 * Each held chunk is one segment of the share's packed layout, documents in order, the
 * lower chunk first:
 *   cu_q[s+1]-cu_q[s] = chunk rows;  off[s] = chunk start within the document;
 *   cu_k[s+1]-cu_k[s] = floor((off[s] + chunk rows) / ratio), the key prefix the chunk's
 *   last row sees;
 *   q_src[s] = batch row of the chunk's first row (share rows cu_q[s].. hold batch rows
 *   q_src[s]..);  k_src[s] = batch key row of the document's first key (share key rows
 *   cu_k[s].. hold batch key rows k_src[s]..).
 * A share id g of segment s is batch key k_src[s] + (g - cu_k[s]).
 * Outputs are HOST arrays owned by the caller, sized for 2*num_docs segments (cu_q and
 * cu_k 2*num_docs+1); *num_segs = 2*num_docs.  Nothing touches the GPU.
 * Errors (CSA_ERR_INVALID, nothing written): a NULL pointer, num_docs < 1, ratio < 1,
 * cp_size < 1, cp_rank outside [0, cp_size), a doc_len < 1 or not divisible by
 * 2*cp_size, totals beyond int32.
 */
csa_status_t csa_cp_plan(int32_t num_docs, const int32_t *doc_len, int32_t ratio, int32_t cp_size,
                         int32_t cp_rank, int32_t *num_segs, int32_t *cu_q, int32_t *cu_k,
                         int32_t *off, int32_t *q_src, int32_t *k_src);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H_ */

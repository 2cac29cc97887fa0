// C ABI of the CSA forward path: host-side validation, then launches on the caller's
// stream.  Every check that the host can make happens before anything is enqueued;
// device data (cu_seqlens, ids) is a documented precondition and is never read here.
#include "../../include/csa.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "launch.h"

namespace {

thread_local char g_err[512] = "";

csa_status_t fail(csa_status_t st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

csa_status_t ok() {
  g_err[0] = '\0';
  return CSA_OK;
}

csa_status_t hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(CSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Layout checks shared by every entry point ("RuntimeError when no segment has compressed
// keys" in the csa.py THD excerpt of the page "[Bug] DSV4 unfused CSA indexer loss uses a
// compressed-only teacher ..." becomes CSA_ERR_INVALID for total_k == 0).
csa_status_t check_layout(const csa_layout_t *L, const char *fn, csa::LaunchLayout *out) {
  if (!L) return fail(CSA_ERR_INVALID, "%s: layout is NULL", fn);
  if (L->num_seqs < 1) return fail(CSA_ERR_INVALID, "%s: num_seqs=%d < 1", fn, L->num_seqs);
  if (L->total_q < 0) return fail(CSA_ERR_INVALID, "%s: total_q=%d < 0", fn, L->total_q);
  if (L->total_k < 1)
    return fail(CSA_ERR_INVALID, "%s: total_k=%d: no segment has compressed keys", fn, L->total_k);
  if (L->max_seqlen_q < 1 || L->max_seqlen_k < 1)
    return fail(CSA_ERR_INVALID, "%s: max_seqlen_q=%d / max_seqlen_k=%d must be >= 1", fn,
                L->max_seqlen_q, L->max_seqlen_k);
  if (L->max_seqlen_q > L->total_q && L->total_q > 0)
    return fail(CSA_ERR_INVALID, "%s: max_seqlen_q=%d > total_q=%d", fn, L->max_seqlen_q, L->total_q);
  if (L->max_seqlen_k > L->total_k)
    return fail(CSA_ERR_INVALID, "%s: max_seqlen_k=%d > total_k=%d", fn, L->max_seqlen_k, L->total_k);
  if (L->compress_ratio < 1)
    return fail(CSA_ERR_INVALID, "%s: compress_ratio=%d < 1", fn, L->compress_ratio);
  if (!L->cu_seqlens_q || !L->cu_seqlens_k)
    return fail(CSA_ERR_INVALID, "%s: cu_seqlens_q / cu_seqlens_k is NULL", fn);
  out->dev.cu_q = L->cu_seqlens_q;
  out->dev.cu_k = L->cu_seqlens_k;
  out->dev.off = L->q_causal_offsets;
  out->dev.cu_q_real = L->cu_seqlens_q_unpadded;
  out->dev.num_seqs = L->num_seqs;
  out->dev.ratio = L->compress_ratio;
  out->num_seqs = L->num_seqs;
  out->total_q = L->total_q;
  out->total_k = L->total_k;
  out->max_seqlen_q = L->max_seqlen_q;
  out->max_seqlen_k = L->max_seqlen_k;
  return CSA_OK;
}

bool dtype_ok(csa_dtype_t dt) { return dt == CSA_F32 || dt == CSA_BF16; }
// the kernels scale logits after taking maxima of unscaled products, so the scale must be
// positive (and finite: a softmax temperature)
bool scale_ok(float s) { return s > 0.f && s <= 3.4e38f; }

int k_eff_of(const csa_layout_t *L, int topk) { return topk < L->max_seqlen_k ? topk : L->max_seqlen_k; }

// Checks shared by the two backward entry points (everything but the workspaces).
csa_status_t check_bwd(const csa_layout_t *L, const char *fn, csa::LaunchLayout *LL, int32_t sparse_loss,
                       const void *q_idx, const void *k_idx, const float *weights, csa_dtype_t dt, int32_t Hi,
                       int32_t Di, const float *scores, int64_t ld_scores, int32_t scores_selected,
                       const int32_t *ids, int32_t k_eff, const float *teacher, int64_t ld_teacher,
                       const float *dq_idx, const float *dweights, const float *dk_idx) {
  csa_status_t st = check_layout(L, fn, LL);
  if (st != CSA_OK) return st;
  if (!q_idx || !k_idx || !weights || !scores || !teacher || !dq_idx || !dweights || !dk_idx)
    return fail(CSA_ERR_INVALID, "%s: a tensor pointer is NULL", fn);
  if (!dtype_ok(dt)) return fail(CSA_ERR_INVALID, "%s: unknown dtype %d", fn, (int)dt);
  if (Hi < 1 || Di < 1) return fail(CSA_ERR_INVALID, "%s: Hi=%d, Di=%d must be >= 1", fn, Hi, Di);
  if (scores_selected && !sparse_loss)
    return fail(CSA_ERR_INVALID, "%s: selected scores need the sparse loss", fn);
  if (ld_scores < (scores_selected ? k_eff : L->max_seqlen_k))
    return fail(CSA_ERR_INVALID, "%s: ld_scores=%lld too small (max_seqlen_k=%d, k_eff=%d)", fn,
                (long long)ld_scores, L->max_seqlen_k, k_eff);
  if (sparse_loss) {
    if (k_eff < 1 || k_eff > L->max_seqlen_k)
      return fail(CSA_ERR_INVALID, "%s: k_eff=%d outside [1, max_seqlen_k=%d]", fn, k_eff, L->max_seqlen_k);
    if (!ids) return fail(CSA_ERR_INVALID, "%s: sparse loss needs ids", fn);
    if (ld_teacher < k_eff)
      return fail(CSA_ERR_INVALID, "%s: ld_teacher=%lld < k_eff=%d", fn, (long long)ld_teacher, k_eff);
  } else if (ld_teacher < L->max_seqlen_k) {
    return fail(CSA_ERR_INVALID, "%s: ld_teacher=%lld < max_seqlen_k=%d", fn, (long long)ld_teacher,
                L->max_seqlen_k);
  }
  if (!csa::indexer_bwd_supported(dt == CSA_BF16, Hi, Di, k_eff, sparse_loss != 0, L->max_seqlen_k))
    return fail(CSA_ERR_UNSUPPORTED, "%s: no kernel for dtype=%d Hi=%d Di=%d k_eff=%d", fn, (int)dt, Hi, Di,
                k_eff);
  return CSA_OK;
}

}  // namespace

extern "C" {

const char *csa_last_error(void) { return g_err; }

int32_t csa_k_eff(const csa_layout_t *L, int32_t topk) {
  if (!L || topk < 0 || L->max_seqlen_k < 1) return -1;
  return k_eff_of(L, topk);
}

csa_status_t csa_indexer_score(const csa_layout_t *L, const void *q_idx, const void *k_idx,
                               const float *weights, csa_dtype_t dt, int32_t Hi, int32_t Di,
                               float idx_scale, float *scores, int64_t ld_scores, void *stream) {
  const char *fn = "csa_indexer_score";
  csa::LaunchLayout LL;
  csa_status_t st = check_layout(L, fn, &LL);
  if (st != CSA_OK) return st;
  if (!q_idx || !k_idx || !weights || !scores)
    return fail(CSA_ERR_INVALID, "%s: a tensor pointer is NULL", fn);
  if (!dtype_ok(dt)) return fail(CSA_ERR_INVALID, "%s: unknown dtype %d", fn, (int)dt);
  if (Hi < 1 || Di < 1) return fail(CSA_ERR_INVALID, "%s: Hi=%d, Di=%d must be >= 1", fn, Hi, Di);
  if (ld_scores < L->max_seqlen_k)
    return fail(CSA_ERR_INVALID, "%s: ld_scores=%lld < max_seqlen_k=%d", fn, (long long)ld_scores,
                L->max_seqlen_k);
  if (!csa::indexer_supported(dt == CSA_BF16, Hi, Di))
    return fail(CSA_ERR_UNSUPPORTED, "%s: no kernel for dtype=%d Hi=%d Di=%d", fn, (int)dt, Hi, Di);
  if (L->total_q == 0) return ok();
  return hip_status(csa::launch_indexer_score(LL, q_idx, k_idx, weights, dt == CSA_BF16, Hi, Di,
                                              idx_scale, scores, ld_scores,
                                              static_cast<hipStream_t>(stream)),
                    fn);
}

csa_status_t csa_topk(const csa_layout_t *L, const float *scores, int64_t ld_scores, int32_t topk,
                      int32_t *ids, float *sel_scores, void *stream) {
  const char *fn = "csa_topk";
  csa::LaunchLayout LL;
  csa_status_t st = check_layout(L, fn, &LL);
  if (st != CSA_OK) return st;
  if (!scores || !ids) return fail(CSA_ERR_INVALID, "%s: a tensor pointer is NULL", fn);
  if (topk < 1) return fail(CSA_ERR_INVALID, "%s: topk=%d < 1", fn, topk);
  if (ld_scores < L->max_seqlen_k)
    return fail(CSA_ERR_INVALID, "%s: ld_scores=%lld < max_seqlen_k=%d", fn, (long long)ld_scores,
                L->max_seqlen_k);
  const int k_eff = k_eff_of(L, topk);
  if (!csa::topk_supported(L->max_seqlen_k, k_eff))
    return fail(CSA_ERR_UNSUPPORTED, "%s: max_seqlen_k=%d exceeds the supported 16384", fn,
                L->max_seqlen_k);
  if (L->total_q == 0) return ok();
  return hip_status(csa::launch_topk(LL, scores, ld_scores, k_eff, ids, sel_scores, static_cast<hipStream_t>(stream)),
                    fn);
}

csa_status_t csa_indexer_topk(const csa_layout_t *L, const void *q_idx, const void *k_idx,
                              const float *weights, csa_dtype_t dt, int32_t Hi, int32_t Di,
                              float idx_scale, int32_t topk, int32_t *ids, float *sel_scores,
                              float *row_lse, void *stream) {
  const char *fn = "csa_indexer_topk";
  csa::LaunchLayout LL;
  csa_status_t st = check_layout(L, fn, &LL);
  if (st != CSA_OK) return st;
  if (!q_idx || !k_idx || !weights || !ids || !sel_scores)
    return fail(CSA_ERR_INVALID, "%s: a tensor pointer is NULL", fn);
  if (!dtype_ok(dt)) return fail(CSA_ERR_INVALID, "%s: unknown dtype %d", fn, (int)dt);
  if (Hi < 1 || Di < 1) return fail(CSA_ERR_INVALID, "%s: Hi=%d, Di=%d must be >= 1", fn, Hi, Di);
  if (topk < 1) return fail(CSA_ERR_INVALID, "%s: topk=%d < 1", fn, topk);
  if (!csa::indexer_topk_supported(dt == CSA_BF16, Hi, Di, L->max_seqlen_k))
    return fail(CSA_ERR_UNSUPPORTED,
                "%s: no fused kernel for dtype=%d Hi=%d Di=%d max_seqlen_k=%d (bf16 (Hi, Di) in {(8,64), "
                "(16,64), (4,128), (8,128), (32,64), (64,64), (16,128), (32,128)} with the block's score "
                "rows in 160 KiB of LDS)",
                fn, (int)dt, Hi, Di, L->max_seqlen_k);
  return hip_status(csa::launch_indexer_topk(LL, q_idx, k_idx, weights, Hi, Di, idx_scale, k_eff_of(L, topk),
                                             ids, sel_scores, row_lse, static_cast<hipStream_t>(stream)),
                    fn);
}

csa_status_t csa_sparse_attn_fwd(const csa_layout_t *L, const void *q, const void *kv,
                                 const void *ckv, const float *sink, const int32_t *ids,
                                 int32_t k_eff, int32_t window, csa_dtype_t dt, int32_t H,
                                 int32_t D, float softmax_scale, void *out, float *lse,
                                 float *lse_nc, float *cmass, void *stream) {
  const char *fn = "csa_sparse_attn_fwd";
  csa::LaunchLayout LL;
  csa_status_t st = check_layout(L, fn, &LL);
  if (st != CSA_OK) return st;
  if (!q || !kv || !ckv || !sink || !out || !lse || !lse_nc)
    return fail(CSA_ERR_INVALID, "%s: a required tensor pointer is NULL", fn);
  if (k_eff < 0 || k_eff > L->max_seqlen_k)
    return fail(CSA_ERR_INVALID, "%s: k_eff=%d outside [0, max_seqlen_k=%d]", fn, k_eff, L->max_seqlen_k);
  if (k_eff > 0 && !ids) return fail(CSA_ERR_INVALID, "%s: ids is NULL with k_eff=%d", fn, k_eff);
  if (window < 0) return fail(CSA_ERR_INVALID, "%s: window=%d < 0", fn, window);
  if (!dtype_ok(dt)) return fail(CSA_ERR_INVALID, "%s: unknown dtype %d", fn, (int)dt);
  if (H < 1 || D < 1) return fail(CSA_ERR_INVALID, "%s: H=%d, D=%d must be >= 1", fn, H, D);
  if (!scale_ok(softmax_scale)) return fail(CSA_ERR_INVALID, "%s: softmax_scale must be finite and > 0", fn);
  if (!csa::attn_supported(dt == CSA_BF16, H, D, k_eff))
    return fail(CSA_ERR_UNSUPPORTED, "%s: no kernel for dtype=%d H=%d D=%d k_eff=%d", fn, (int)dt, H, D, k_eff);
  if (L->total_q == 0) return ok();
  return hip_status(csa::launch_sparse_attn(LL, q, kv, ckv, sink, ids, k_eff, window, dt == CSA_BF16, H,
                                            D, softmax_scale, out, lse, lse_nc, cmass,
                                            static_cast<hipStream_t>(stream)),
                    fn);
}

csa_status_t csa_indexer_teacher_kl(const csa_layout_t *L, int32_t sparse_loss, const float *scores,
                                    int64_t ld_scores, int32_t scores_selected, const int32_t *ids,
                                    int32_t k_eff,
                                    const float *cmass, const void *q, const void *ckv,
                                    const float *lse_nc, csa_dtype_t dt, int32_t H, int32_t D,
                                    float softmax_scale, int32_t per_token_loss, float *teacher,
                                    int64_t ld_teacher, float *kl_row, float *loss, void *stream) {
  const char *fn = "csa_indexer_teacher_kl";
  csa::LaunchLayout LL;
  csa_status_t st = check_layout(L, fn, &LL);
  if (st != CSA_OK) return st;
  if (!scores || !kl_row || !loss) return fail(CSA_ERR_INVALID, "%s: scores/kl_row/loss is NULL", fn);
  if (scores_selected && !sparse_loss)
    return fail(CSA_ERR_INVALID, "%s: selected scores need the sparse loss", fn);
  const int need_ld = scores_selected ? k_eff : L->max_seqlen_k;
  if (ld_scores < need_ld)
    return fail(CSA_ERR_INVALID, "%s: ld_scores=%lld < %d", fn, (long long)ld_scores, need_ld);
  if (sparse_loss) {
    if (k_eff < 1 || k_eff > L->max_seqlen_k)
      return fail(CSA_ERR_INVALID, "%s: k_eff=%d outside [1, max_seqlen_k=%d]", fn, k_eff, L->max_seqlen_k);
    if (!ids || !cmass) return fail(CSA_ERR_INVALID, "%s: sparse loss needs ids and cmass", fn);
    if (k_eff > 4096) return fail(CSA_ERR_UNSUPPORTED, "%s: k_eff=%d above the supported 4096", fn, k_eff);
    if (teacher && ld_teacher < k_eff)
      return fail(CSA_ERR_INVALID, "%s: ld_teacher=%lld < k_eff=%d", fn, (long long)ld_teacher, k_eff);
  } else {
    if (!q || !ckv || !lse_nc) return fail(CSA_ERR_INVALID, "%s: dense loss needs q, ckv and lse_nc", fn);
    if (!scale_ok(softmax_scale)) return fail(CSA_ERR_INVALID, "%s: softmax_scale must be finite and > 0", fn);
    if (!dtype_ok(dt)) return fail(CSA_ERR_INVALID, "%s: unknown dtype %d", fn, (int)dt);
    if (H < 1 || D < 1) return fail(CSA_ERR_INVALID, "%s: H=%d, D=%d must be >= 1", fn, H, D);
    if (teacher && ld_teacher < L->max_seqlen_k)
      return fail(CSA_ERR_INVALID, "%s: ld_teacher=%lld < max_seqlen_k=%d", fn, (long long)ld_teacher,
                  L->max_seqlen_k);
    if (!csa::dense_teacher_supported(dt == CSA_BF16, H, D, L->max_seqlen_k))
      return fail(CSA_ERR_UNSUPPORTED, "%s: no dense kernel for dtype=%d H=%d D=%d max_seqlen_k=%d", fn,
                  (int)dt, H, D, L->max_seqlen_k);
  }
  return hip_status(csa::launch_teacher_kl(LL, sparse_loss != 0, scores, ld_scores, scores_selected != 0,
                                           ids, k_eff, cmass, q,
                                           ckv, lse_nc, dt == CSA_BF16, H, D, softmax_scale,
                                           per_token_loss != 0, teacher, ld_teacher, kl_row, loss,
                                           static_cast<hipStream_t>(stream)),
                    fn);
}

csa_status_t csa_sparse_attn_kl_fwd(const csa_layout_t *L, const void *q, const void *kv, const void *ckv,
                                    const float *sink, const int32_t *ids, int32_t k_eff, int32_t window,
                                    csa_dtype_t dt, int32_t H, int32_t D, float softmax_scale,
                                    const float *scores, int64_t ld_scores, int32_t scores_selected,
                                    int32_t per_token_loss, void *out, float *lse, float *lse_nc,
                                    float *cmass, float *teacher, int64_t ld_teacher, float *kl_row,
                                    float *loss, void *stream) {
  const char *fn = "csa_sparse_attn_kl_fwd";
  csa::LaunchLayout LL;
  csa_status_t st = check_layout(L, fn, &LL);
  if (st != CSA_OK) return st;
  if (!q || !kv || !ckv || !sink || !ids || !out || !lse || !lse_nc || !cmass || !scores || !kl_row)
    return fail(CSA_ERR_INVALID, "%s: a required tensor pointer is NULL", fn);
  if (k_eff < 1 || k_eff > L->max_seqlen_k)
    return fail(CSA_ERR_INVALID, "%s: k_eff=%d outside [1, max_seqlen_k=%d]", fn, k_eff, L->max_seqlen_k);
  if (window < 0) return fail(CSA_ERR_INVALID, "%s: window=%d < 0", fn, window);
  if (!dtype_ok(dt)) return fail(CSA_ERR_INVALID, "%s: unknown dtype %d", fn, (int)dt);
  if (H < 1 || D < 1) return fail(CSA_ERR_INVALID, "%s: H=%d, D=%d must be >= 1", fn, H, D);
  const int need_ld = scores_selected ? k_eff : L->max_seqlen_k;
  if (ld_scores < need_ld)
    return fail(CSA_ERR_INVALID, "%s: ld_scores=%lld < %d", fn, (long long)ld_scores, need_ld);
  if (teacher && ld_teacher < k_eff)
    return fail(CSA_ERR_INVALID, "%s: ld_teacher=%lld < k_eff=%d", fn, (long long)ld_teacher, k_eff);
  if (!scale_ok(softmax_scale)) return fail(CSA_ERR_INVALID, "%s: softmax_scale must be finite and > 0", fn);
  if (!csa::attn_supported(dt == CSA_BF16, H, D, k_eff))
    return fail(CSA_ERR_UNSUPPORTED, "%s: no kernel for dtype=%d H=%d D=%d k_eff=%d", fn, (int)dt, H, D, k_eff);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (scores_selected && csa::attn_kl_fused_supported(LL, dt == CSA_BF16, H, D, k_eff, window)) {
    // one attention launch that also finishes the teacher and the KL, then the loss
    if (L->total_q > 0) {
      const csa::KlArgs kla{scores, ld_scores, teacher, ld_teacher, kl_row};
      st = hip_status(csa::launch_sparse_attn_kl(LL, q, kv, ckv, sink, ids, k_eff, window, H, D, softmax_scale,
                                                 out, lse, lse_nc, cmass, kla, hs),
                      fn);
      if (st != CSA_OK) return st;
    }
    if (!loss) return ok();
    return hip_status(csa::launch_loss_reduce(kl_row, L->total_q, per_token_loss != 0, loss, hs), fn);
  }
  if (L->total_q > 0) {
    st = hip_status(csa::launch_sparse_attn(LL, q, kv, ckv, sink, ids, k_eff, window, dt == CSA_BF16, H, D,
                                            softmax_scale, out, lse, lse_nc, cmass, hs),
                    fn);
    if (st != CSA_OK) return st;
  }
  return hip_status(csa::launch_teacher_kl(LL, true, scores, ld_scores, scores_selected != 0, ids, k_eff, cmass,
                                           nullptr, nullptr, nullptr, dt == CSA_BF16, H, D, softmax_scale,
                                           per_token_loss != 0, teacher, ld_teacher, kl_row, loss, hs),
                    fn);
}

csa_status_t csa_loss_reduce(const float *kl_row, int32_t total_q, int32_t per_token_loss, float *loss,
                             void *stream) {
  const char *fn = "csa_loss_reduce";
  if (!loss) return fail(CSA_ERR_INVALID, "%s: loss is NULL", fn);
  if (total_q < 0) return fail(CSA_ERR_INVALID, "%s: total_q=%d < 0", fn, total_q);
  if (total_q > 0 && !kl_row) return fail(CSA_ERR_INVALID, "%s: kl_row is NULL", fn);
  return hip_status(csa::launch_loss_reduce(kl_row, total_q, per_token_loss != 0, loss,
                                            static_cast<hipStream_t>(stream)),
                    fn);
}

csa_status_t csa_indexer_loss_bwd(const csa_layout_t *L, int32_t sparse_loss, const void *q_idx,
                                  const void *k_idx, const float *weights, csa_dtype_t dt, int32_t Hi,
                                  int32_t Di, float idx_scale, const float *scores, int64_t ld_scores,
                                  int32_t scores_selected, const int32_t *ids, int32_t k_eff,
                                  const float *teacher,
                                  int64_t ld_teacher, float grad_loss, int32_t per_token_loss,
                                  float *grad_scores, int64_t ld_grad, float *dq_idx, float *dweights,
                                  float *dk_idx, void *workspace, int64_t workspace_bytes,
                                  void *stream) {
  const char *fn = "csa_indexer_loss_bwd";
  csa::LaunchLayout LL;
  csa_status_t st = check_bwd(L, fn, &LL, sparse_loss, q_idx, k_idx, weights, dt, Hi, Di, scores, ld_scores,
                              scores_selected, ids, k_eff, teacher, ld_teacher, dq_idx, dweights, dk_idx);
  if (st != CSA_OK) return st;
  if (!grad_scores) return fail(CSA_ERR_INVALID, "%s: grad_scores is NULL", fn);
  if (ld_grad < L->max_seqlen_k)
    return fail(CSA_ERR_INVALID, "%s: ld_grad=%lld < max_seqlen_k=%d", fn, (long long)ld_grad, L->max_seqlen_k);
  const int64_t need = csa::indexer_bwd_workspace_bytes(L->num_seqs, L->total_k, L->max_seqlen_q,
                                                        L->max_seqlen_k, Di);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(CSA_ERR_INVALID, "%s: workspace of %lld bytes given, %lld needed", fn,
                (long long)(workspace ? workspace_bytes : 0), (long long)need);
  const float gscale = per_token_loss ? grad_loss : (L->total_q > 0 ? grad_loss / (float)L->total_q : 0.f);
  return hip_status(csa::launch_indexer_loss_bwd(LL, sparse_loss != 0, q_idx, k_idx, weights, Hi, Di,
                                                  idx_scale, scores, ld_scores, scores_selected != 0, ids,
                                                  k_eff, teacher,
                                                  ld_teacher, gscale, grad_scores, ld_grad, dq_idx,
                                                  dweights, dk_idx, workspace,
                                                  static_cast<hipStream_t>(stream)),
                    fn);
}

csa_status_t csa_indexer_loss_bwd_noalloc(const csa_layout_t *L, int32_t sparse_loss, const void *q_idx,
                                          const void *k_idx, const float *weights, csa_dtype_t dt, int32_t Hi,
                                          int32_t Di, float idx_scale, const float *scores, int64_t ld_scores,
                                          int32_t scores_selected, const int32_t *ids, int32_t k_eff,
                                          const float *teacher, int64_t ld_teacher, float grad_loss,
                                          int32_t per_token_loss, float *dq_idx, float *dweights, float *dk_idx,
                                          void *stream) {
  const char *fn = "csa_indexer_loss_bwd_noalloc";
  csa::LaunchLayout LL;
  csa_status_t st = check_bwd(L, fn, &LL, sparse_loss, q_idx, k_idx, weights, dt, Hi, Di, scores, ld_scores,
                              scores_selected, ids, k_eff, teacher, ld_teacher, dq_idx, dweights, dk_idx);
  if (st != CSA_OK) return st;
  const csa::NoallocPlan plan = csa::noalloc_plan(L->num_seqs, L->total_q, L->total_k, L->max_seqlen_q,
                                                  L->max_seqlen_k, Di);
  if (plan.bytes > csa::NOALLOC_SCRATCH_BYTES)
    return fail(CSA_ERR_INVALID,
                "%s: this layout needs %lld bytes of scratch (score gradients and dk partials), above the "
                "library's %lld; use csa_indexer_loss_bwd with caller workspaces",
                fn, (long long)plan.bytes, (long long)csa::NOALLOC_SCRATCH_BYTES);
  void *base = nullptr;
  st = hip_status(csa::noalloc_scratch_ptr(&base), fn);
  if (st != CSA_OK) return st;
  char *b = static_cast<char *>(base);
  const float gscale = per_token_loss ? grad_loss : (L->total_q > 0 ? grad_loss / (float)L->total_q : 0.f);
  return hip_status(csa::launch_indexer_loss_bwd(LL, sparse_loss != 0, q_idx, k_idx, weights, Hi, Di,
                                                  idx_scale, scores, ld_scores, scores_selected != 0, ids,
                                                  k_eff, teacher, ld_teacher, gscale,
                                                  reinterpret_cast<float *>(b), plan.ld_grad, dq_idx,
                                                  dweights, dk_idx, b + plan.ws_offset,
                                                  static_cast<hipStream_t>(stream)),
                    fn);
}

int64_t csa_indexer_loss_bwd_workspace(const csa_layout_t *L, int32_t Hi, int32_t Di) {
  csa::LaunchLayout LL;
  if (check_layout(L, "csa_indexer_loss_bwd_workspace", &LL) != CSA_OK) return -1;
  if (!csa::indexer_bwd_supported(true, Hi, Di, 1, true, 1)) {
    fail(CSA_ERR_UNSUPPORTED, "csa_indexer_loss_bwd_workspace: no kernel for Hi=%d Di=%d", Hi, Di);
    return -1;
  }
  ok();
  return csa::indexer_bwd_workspace_bytes(L->num_seqs, L->total_k, L->max_seqlen_q, L->max_seqlen_k, Di);
}

csa_status_t csa_cp_plan(int32_t num_docs, const int32_t *doc_len, int32_t ratio, int32_t cp_size,
                         int32_t cp_rank, int32_t *num_segs, int32_t *cu_q, int32_t *cu_k,
                         int32_t *off, int32_t *q_src, int32_t *k_src) {
  const char *fn = "csa_cp_plan";
  if (!doc_len || !num_segs || !cu_q || !cu_k || !off || !q_src || !k_src)
    return fail(CSA_ERR_INVALID, "%s: NULL argument", fn);
  if (num_docs < 1 || ratio < 1 || cp_size < 1)
    return fail(CSA_ERR_INVALID, "%s: num_docs=%d ratio=%d cp_size=%d must be >= 1", fn, num_docs,
                ratio, cp_size);
  if (cp_rank < 0 || cp_rank >= cp_size)
    return fail(CSA_ERR_INVALID, "%s: cp_rank=%d outside [0, %d)", fn, cp_rank, cp_size);
  const int64_t nchunk = 2 * (int64_t)cp_size;
  int64_t tq = 0, tk = 0, bq = 0, bk = 0;
  for (int32_t d = 0; d < num_docs; ++d) {
    if (doc_len[d] < 1 || doc_len[d] % nchunk != 0)
      return fail(CSA_ERR_INVALID, "%s: doc_len[%d]=%d is not a positive multiple of 2*cp_size=%lld",
                  fn, d, doc_len[d], (long long)nchunk);
    const int64_t c = doc_len[d] / nchunk;
    tq += 2 * c;
    tk += (((int64_t)cp_rank + 1) * c) / ratio + ((nchunk - cp_rank) * c) / ratio;
    bq += doc_len[d];
    bk += doc_len[d] / ratio;
  }
  if (tq > INT32_MAX || tk > INT32_MAX || bq > INT32_MAX || bk > INT32_MAX)
    return fail(CSA_ERR_INVALID, "%s: totals exceed int32", fn);
  int32_t s = 0, row = 0, key = 0;
  cu_q[0] = cu_k[0] = 0;
  int64_t doc_row = 0, doc_key = 0;
  for (int32_t d = 0; d < num_docs; ++d) {
    const int32_t c = (int32_t)(doc_len[d] / nchunk);
    const int32_t held[2] = {cp_rank, (int32_t)(nchunk - 1 - cp_rank)};
    for (int32_t h = 0; h < 2; ++h) {
      const int32_t start = held[h] * c;
      const int32_t nkeys = (start + c) / ratio;
      off[s] = start;
      q_src[s] = (int32_t)(doc_row + start);
      k_src[s] = (int32_t)doc_key;
      row += c;
      key += nkeys;
      cu_q[s + 1] = row;
      cu_k[s + 1] = key;
      ++s;
    }
    doc_row += doc_len[d];
    doc_key += doc_len[d] / ratio;
  }
  *num_segs = s;
  return ok();
}

}  // extern "C"

// Internal launch interface between the C-ABI layer (csa_api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "../../include/csa.h"
#include "kernels/common.h"
#include "kernels/sparse_kl.h"

namespace csa {

struct LaunchLayout {
  LayoutDev dev;
  int num_seqs, total_q, total_k, max_seqlen_q, max_seqlen_k;
};

hipError_t launch_indexer_score(const LaunchLayout &L, const void *q_idx, const void *k_idx,
                                const float *weights, bool bf16, int Hi, int Di, float idx_scale,
                                float *scores, int64_t ld, hipStream_t st);

hipError_t launch_topk(const LaunchLayout &L, const float *scores, int64_t ld, int k_eff,
                       int32_t *ids, float *sel /* NULL: ids only */, hipStream_t st);

hipError_t launch_sparse_attn(const LaunchLayout &L, const void *q, const void *kv,
                              const void *ckv, const float *sink, const int32_t *ids, int k_eff,
                              int window, bool bf16, int H, int D, float scale, void *out,
                              float *lse, float *lse_nc, float *cmass, hipStream_t st);

// the D = 512 workgroup attention (P.V split over the output columns; bf16, H <= 128)
hipError_t launch_sparse_attn_wide(const LaunchLayout &L, const void *q, const void *kv, const void *ckv,
                                   const float *sink, const int32_t *ids, int k_eff, int window, int H,
                                   float scale, void *out, float *lse, float *lse_nc, float *cmass,
                                   hipStream_t st);

// its first pass: lse and lse_nc of every row (also bf16, D = 512, H <= 128)
hipError_t launch_sparse_attn_wide_lse(const LaunchLayout &L, const void *q, const void *kv, const void *ckv,
                                       const float *sink, const int32_t *ids, int k_eff, int window, int H,
                                       float scale, float *lse, float *lse_nc, hipStream_t st);

// attention whose epilogue also finishes the sparse teacher and KL (kl_row, teacher)
// from the selected scores; only for shapes where attn_kl_fused_supported holds
hipError_t launch_sparse_attn_kl(const LaunchLayout &L, const void *q, const void *kv,
                                 const void *ckv, const float *sink, const int32_t *ids, int k_eff,
                                 int window, int H, int D, float scale, void *out, float *lse,
                                 float *lse_nc, float *cmass, const KlArgs &kla, hipStream_t st);
// loss[0] = sum_t kl_row[t] (/ T unless per_token), one workgroup, fixed order
hipError_t launch_loss_reduce(const float *kl_row, int T, bool per_token, float *loss, hipStream_t st);

hipError_t launch_teacher_kl(const LaunchLayout &L, bool sparse, const float *scores, int64_t ld,
                             bool selected, const int32_t *ids, int k_eff, const float *cmass, const void *q,
                             const void *ckv, const float *lse_nc, bool bf16, int H, int D,
                             float scale, bool per_token, float *teacher, int64_t ld_teacher,
                             float *kl_row, float *loss /* NULL: kl_row only */, hipStream_t st);

hipError_t launch_indexer_loss_bwd(const LaunchLayout &L, bool sparse, const void *q_idx,
                                  const void *k_idx, const float *weights, int Hi, int Di,
                                  float idx_scale, const float *scores, int64_t ld_scores,
                                  bool selected, const int32_t *ids, int k_eff, const float *teacher,
                                  int64_t ld_teacher, float grad_scale, float *grad, int64_t ld_grad,
                                  float *dq, float *dw, float *dk, void *workspace, hipStream_t st);
// device workspace of the indexer-loss backward (dk partials per token-block chunk; 0: none)
int64_t indexer_bwd_workspace_bytes(int num_seqs, int total_k, int max_seqlen_q, int max_seqlen_k, int Di);

// the no-allocation backward: G and the dk partials in the library's static device scratch
constexpr int64_t NOALLOC_SCRATCH_BYTES = CSA_NOALLOC_SCRATCH_BYTES;
struct NoallocPlan {
  int64_t ld_grad;    // row stride of G (floats)
  int64_t ws_offset;  // byte offset of the dk partials
  int64_t bytes;      // scratch bytes the call needs
};
NoallocPlan noalloc_plan(int num_seqs, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int Di);
// device address of this device's scratch (looked up on the first call per device)
hipError_t noalloc_scratch_ptr(void **ptr);

hipError_t launch_indexer_topk(const LaunchLayout &L, const void *q_idx, const void *k_idx,
                               const float *weights, int Hi, int Di, float idx_scale, int k_eff,
                               int32_t *ids, float *sel, float *lse, hipStream_t st);

// shape support tables (host side, used by validation before any launch)
bool indexer_supported(bool bf16, int Hi, int Di);
bool indexer_topk_supported(bool bf16, int Hi, int Di, int max_seqlen_k);
bool topk_supported(int max_seqlen_k, int k_eff);
bool attn_supported(bool bf16, int H, int D, int k_eff);
bool attn_kl_fused_supported(const LaunchLayout &L, bool bf16, int H, int D, int k_eff, int window);
bool dense_teacher_supported(bool bf16, int H, int D, int max_seqlen_k);
bool indexer_bwd_supported(bool bf16, int Hi, int Di, int k_eff, bool sparse, int max_seqlen_k);

}  // namespace csa

"""The compressed-only teacher of the unfused Megatron-LM path, written from its
description -- TEST INFRASTRUCTURE ONLY (used as a pin of the oracle's teacher).

[I5776, section "2. The small operators recompute a compressed-only softmax", the
t-hat equation, and the dsa.py ``compute_dsa_indexer_loss`` excerpt]: QK scores over
the whole [B*np, sq, sk] rectangle scaled by softmax_scale; an additive causal mask
and (sparse loss) an additive -inf index mask built by scattering 0 at the top-k
columns; rows with no visible key zeroed before the softmax and after it; a softmax
per head over the key axis; the sum over heads; one L1 normalisation clamped at 1e-10.

The paper teacher of the oracle must reduce to this when the window is empty and the
sink is -inf (then every Z_h holds only the compressed terms).  The two routines are
deliberately organised differently: this one works on whole masked matrices, the
oracle works row by row on gathered keys.
"""
import numpy as np


def compressed_only_teacher(q, k, causal_mask, topk_local, scale, sparse):
    """q: [sq, H, D]; k: [sk, D] (one KV head broadcast to every head);
    causal_mask: [sq, sk] additive (0 or -inf); topk_local: [sq, kk] local column ids
    (-1 allowed, ignored) or None; returns the teacher matrix [sq, sk]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    sq, H, D = q.shape
    sk = k.shape[0]
    scores = np.einsum("shd,kd->hsk", q, k) * float(scale)          # [H, sq, sk]
    scores = scores + causal_mask[None, :, :]
    if sparse:
        index_mask = np.full((sq, sk), -np.inf)
        for s in range(sq):
            for j in topk_local[s]:
                if j >= 0:
                    index_mask[s, j] = 0.0
        scores = scores + index_mask[None, :, :]
    row_valid = np.any(causal_mask > -np.inf, axis=-1)               # [sq]
    scores = np.where(row_valid[None, :, None], scores, 0.0)
    m = np.max(scores, axis=-1, keepdims=True)
    e = np.exp(scores - m)
    probs = e / np.sum(e, axis=-1, keepdims=True)
    probs = probs * row_valid[None, :, None]
    summed = probs.sum(axis=0)                                       # [sq, sk]
    return summed / np.maximum(summed.sum(axis=-1, keepdims=True), 1e-10)

"""Oracle pins of context-parallel (CP) scoring on one rank's share ([PR8539], item 2 and
test plan): a query chunk scored against its document's cropped key prefix with the
chunk's absolute causal offset gives every row the scores and the top-k of the whole
document run; with the offsets removed (top-left alignment, offset 0) the selection
changes -- the pull request's negative control.  With the prefix cropped at the chunk
end, the bottom-right default of the layout gives the same offsets.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests import cp_rule, tiny

RATIO = 2


def _share_problem(P, docs, cp, rank, offsets="explicit"):
    """The rank's share as an oracle problem, plus the per-segment (batch_row0, batch_key0)."""
    segs = cp_rule.share(docs, RATIO, cp, rank)
    rows, keys, cq, ck, off = [], [], [0], [0], []
    for (_, a, c, nk, r0, k0) in segs:
        rows += range(r0, r0 + c)
        keys += range(k0, k0 + nk)
        cq.append(cq[-1] + c)
        ck.append(ck[-1] + nk)
        off.append(a)
    o = {"explicit": np.asarray(off), "top-left": np.zeros(len(off)), "default": None}[offsets]
    L = oracle.Layout(cu_q=np.asarray(cq), cu_k=np.asarray(ck), ratio=RATIO,
                      off=None if o is None else o.astype(np.int64))
    S = oracle.Problem(layout=L, q=P.q[rows], kv=P.kv[rows], ckv=P.ckv[keys], q_idx=P.q_idx[rows],
                       k_idx=P.k_idx[keys], weights=P.weights[rows], sink=P.sink, topk=P.topk,
                       window=P.window, scale=P.scale, idx_scale=P.idx_scale)
    return S, segs, rows


def _compare(P, docs, cp, rank, offsets):
    """Number of share rows whose selection differs from the whole-document run."""
    S, segs, rows = _share_problem(P, docs, cp, rank, offsets)
    k_eff = oracle.k_eff_of(P.layout, P.topk)
    differ = 0
    for t_s, t in enumerate(rows):
        g_s = oracle.row_geometry(S.layout, t_s)
        g = oracle.row_geometry(P.layout, t)
        s_idx = g_s.seg
        sc_s = oracle.indexer_scores_row(S.q_idx[t_s], S.weights[t_s],
                                         S.k_idx[g_s.k_base:int(S.layout.cu_k[s_idx + 1])],
                                         S.idx_scale, g_s.n_valid)
        sc = oracle.indexer_scores_row(P.q_idx[t], P.weights[t],
                                       P.k_idx[g.k_base:int(P.layout.cu_k[g.seg + 1])],
                                       P.idx_scale, g.n_valid)
        ids_s = oracle.topk_row(sc_s, g_s.n_valid, k_eff, g_s.k_base)
        ids = oracle.topk_row(sc, g.n_valid, k_eff, g.k_base)
        k0 = segs[s_idx][5]
        mapped = np.where(ids_s >= 0, ids_s - g_s.k_base + k0, -1)
        if offsets != "top-left":
            assert g_s.n_valid == g.n_valid, (t, g_s.n_valid, g.n_valid)
            np.testing.assert_array_equal(sc_s[:g_s.n_valid], sc[:g.n_valid])
        differ += int(not np.array_equal(mapped, ids))
    return differ


CASES = [((48,), 1, 0), ((48,), 2, 0), ((48,), 2, 1), ((16, 32), 2, 0), ((16, 32), 2, 1)]


@pytest.mark.parametrize("docs,cp,rank", CASES)
@pytest.mark.parametrize("offsets", ["explicit", "default"])
def test_share_selects_what_the_whole_document_selects(docs, cp, rank, offsets):
    P = tiny.problem(seg_lens=docs, ratio=RATIO, Hi=3, Di=6, topk=4, window=3, seed=21)
    assert _compare(P, docs, cp, rank, offsets) == 0


@pytest.mark.parametrize("docs,cp,rank", CASES)
def test_negative_control_top_left_changes_the_selection(docs, cp, rank):
    P = tiny.problem(seg_lens=docs, ratio=RATIO, Hi=3, Di=6, topk=4, window=3, seed=21)
    assert _compare(P, docs, cp, rank, "top-left") > 0

"""Plain CPU oracle for the compressed-sparse-attention (CSA) forward hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or runs this
module: only the test suite, the smoke check and the benchmark's cpu_baseline leg do.
It shares no code with the HIP library or its Python binding and imports nothing from
them.  It takes plain NumPy arrays (the exact values the GPU reads, widened to float64)
and computes every step per query row, in float64, straight from the definitions.

Sources, cited by tag throughout:

[I5776]  the page "[Bug] DSV4 unfused CSA indexer loss uses a compressed-only teacher
         instead of the full CSA attention distribution" (Megatron-LM issue 5776).  It
         exists in two copies: a markdown mirror, and a GitHub copy that adds the
         Megatron-LM code excerpts (csa.py SBHD causal-mask excerpt, csa.py THD excerpt,
         dsa.py ``compute_dsa_indexer_loss`` excerpt, csa.py sparse-attention excerpt,
         dsa_kernels.py fused-path excerpt) and the discussion thread (the proposal
         comment that defines u_h, l_h and p_hj; the review comment on the KL contract
         and the loss divisor).
[PR8539] the page "Megatron-LM pull request 8539" (cuDNN frontend 1.26 changed the top-k
         id locality and the default causal alignment), items 1 and 2 and its test plan.

Readings where the pages are silent or ambiguous are marked READING and listed with
their justification in the design document.  One function has no pin from the pages
and is marked "parity unpinned": ``window_rows`` (the pages use the window ids
without defining them).

Notation (per query row t of segment s):
    r      = t - cu_q[s]                 local query index
    i      = r + 1 + off[s]              1-based absolute position (bottom-right aligned)
    S_k(s) = cu_k[s+1] - cu_k[s]         compressed keys of the segment
    n_valid(t) = clamp(floor(i / ratio), 0, S_k(s))   causally visible compressed keys
    k_eff  = min(topk, max_s S_k(s))     selection width
    K_t    = min(k_eff, n_valid(t))      selected keys of row t
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

NEG_INF = -np.inf
EPS_L1 = 1e-10   # teacher L1 clamp  [I5776, dsa.py excerpt: sum(...).clamp(min=1e-10)]
EPS_LOG = 1e-10  # KL log epsilon    [I5776, dsa.py excerpt: log(x + 1e-10)]; kept as-is per the
                 # review comment's "KL numerical contract" section


# --------------------------------------------------------------------------------------
# Layout and row geometry
# --------------------------------------------------------------------------------------
@dataclass
class Layout:
    """Packed (THD) layout; a BSHD batch is the special case cu_q = [0, S, 2S, ...].

    cu_q : int array [B+1]  query row boundaries (row t belongs to segment s iff
                             cu_q[s] <= t < cu_q[s+1])
    cu_k : int array [B+1]  compressed-key row boundaries of each segment
    ratio: int >= 1         compression ratio
    off  : int array [B] or None  per-segment causal offsets; None means the
                             bottom-right default of ``default_offsets``.
    cu_q_real : int array [B+1] or None  real (unpadded) query boundaries of a batch
                             whose segments carry trailing padding rows; None: no padding.
    """
    cu_q: np.ndarray
    cu_k: np.ndarray
    ratio: int
    off: np.ndarray | None = None
    cu_q_real: np.ndarray | None = None

    @property
    def num_seqs(self) -> int:
        return len(self.cu_q) - 1

    @property
    def total_q(self) -> int:
        return int(self.cu_q[-1])

    @property
    def total_k(self) -> int:
        return int(self.cu_k[-1])

    @property
    def max_seqlen_k(self) -> int:
        return int(np.max(np.diff(self.cu_k))) if self.num_seqs else 0

    def offsets(self) -> np.ndarray:
        if self.off is None:
            return default_offsets(self.cu_q, self.cu_k, self.ratio)
        return np.asarray(self.off, dtype=np.int64)


def default_offsets(cu_q, cu_k, ratio) -> np.ndarray:
    """Bottom-right causal alignment per segment: seqlen_k * ratio - seqlen_q.

    [PR8539, item 2 "Causal offsets"]: the bottom-right alignment is
    seqlen_k * ratio - seqlen_q.  The same item later writes the THD offsets as
    segment_k_lengths - segment_q_lengths without the ratio; READING: the ratio is
    kept, because without it rows of a full document would see almost no keys, which
    contradicts the compressed causal mask of [I5776, csa.py SBHD excerpt].
    """
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    return np.diff(cu_k) * int(ratio) - np.diff(cu_q)


def compressed_cu_seqlens(cu_q, ratio) -> np.ndarray:
    """cu_k = [0, cumsum(seg_len_q // ratio)]  [I5776, csa.py THD excerpt: the loss path
    rebuilds the compressed cu_seqlens from the query segment lengths]."""
    seg = np.diff(np.asarray(cu_q, dtype=np.int64))
    return np.concatenate([[0], np.cumsum(seg // int(ratio))]).astype(np.int64)


@dataclass
class RowGeom:
    seg: int        # segment s
    local: int      # r
    pos: int        # i (1-based absolute position)
    n_valid: int    # visible compressed keys
    k_base: int     # cu_k[s]  (global id of local key 0)
    q_start: int    # cu_q[s]
    padding: bool = False   # row past its segment's real length (left out of the loss)


def segment_of_row(cu_q, t: int) -> int:
    """Segment s with cu_q[s] <= t < cu_q[s+1] (the role of ``batch_of_row`` in
    [I5776, dsa_kernels.py fused-path excerpt]).  Found by a plain scan."""
    for s in range(len(cu_q) - 1):
        if cu_q[s] <= t < cu_q[s + 1]:
            return s
    raise IndexError(f"row {t} outside every segment")


def row_geometry(L: Layout, t: int) -> RowGeom:
    """Causal geometry of query row t.

    [I5776, csa.py SBHD excerpt]: with 1-based positions, query position i masks every
    compressed key j with j >= i // compress_ratio, so it sees keys 0 .. i//ratio - 1.
    [PR8539, item 2]: in a packed batch each segment carries an offset that aligns the
    mask bottom-right; i = r + 1 + off[s].
    READING: a non-positive numerator means no visible key (clamp at 0), and a row never
    sees past its own segment's keys (clamp at S_k(s)).

    Padding ([I5776, dsa_kernels.py fused-path excerpt, step 4b]): when CUDA-graph padding
    makes cu_q cover every physical row, the unpadded boundaries give each segment's real
    length, and a row whose position in its segment is at or past that length is padding
    (every row of a trailing dummy segment of real length 0 is).
    """
    s = segment_of_row(L.cu_q, t)
    r = t - int(L.cu_q[s])
    i = r + 1 + int(L.offsets()[s])
    s_k = int(L.cu_k[s + 1] - L.cu_k[s])
    n = i // L.ratio if i > 0 else 0
    n = max(0, min(n, s_k))
    padding = False
    if L.cu_q_real is not None:
        padding = r >= int(L.cu_q_real[s + 1] - L.cu_q_real[s])
    return RowGeom(seg=s, local=r, pos=i, n_valid=n, k_base=int(L.cu_k[s]), q_start=int(L.cu_q[s]),
                   padding=padding)


def k_eff_of(L: Layout, topk: int) -> int:
    """k = min(index_topk, max compressed length)  [I5776, csa.py SBHD excerpt
    ``min(index_topk, n_compressed)`` and THD excerpt ``min(index_topk,
    max_seqlen_compressed_idx)``]."""
    return min(int(topk), L.max_seqlen_k)


# --------------------------------------------------------------------------------------
# Step 1: Lightning-Indexer scores
# --------------------------------------------------------------------------------------
def indexer_weight_scale(w_row, idx_scale, exact: bool = False) -> np.ndarray:
    """fp32(weights) * fp32(indexer softmax scale), rounded to fp32 (exact=True keeps the
    float64 product; only the finite-difference pins of the backward use it).

    [I5776, csa.py SBHD excerpt]: the indexer scale is folded into the per-head weights as
    ``weights.float() * indexer.softmax_scale`` before the loss call.  READING: the
    product is formed in fp32 (the SBHD form; the review comment notes that the
    rounding point can change selection near a tie)."""
    if exact:
        return np.asarray(w_row, dtype=np.float64) * float(np.float32(idx_scale))
    return (np.asarray(w_row, dtype=np.float32) * np.float32(idx_scale)).astype(np.float32)


def indexer_scores_row(q_idx_t, w_t, k_idx_seg, idx_scale, n_valid, exact_ws: bool = False) -> np.ndarray:
    """Scores I[t, j] for all local keys j of the row's segment.

    READING (the pages do not print the score formula; they show the weight/scale folding
    and a per-indexer-head intermediate of shape [Sq, B, H_index, Sk]):
        I[t, j] = sum_h  ws[h] * max(0, q_idx[t, h, :] . k_idx[j, :])     for j < n_valid
        I[t, j] = -inf                                                     otherwise
    with ws = fp32(w[t, h] * s_idx).  One indexer key row is shared by all indexer
    heads (the excerpts squeeze a singleton head axis of k_indexer).

    q_idx_t: [Hi, Di]; w_t: [Hi]; k_idx_seg: [S_k, Di] (the segment's keys).
    Returns float64 [S_k].
    """
    q = np.asarray(q_idx_t, dtype=np.float64)
    k = np.asarray(k_idx_seg, dtype=np.float64)
    ws = indexer_weight_scale(w_t, idx_scale, exact_ws).astype(np.float64)
    s_k = k.shape[0]
    out = np.full(s_k, NEG_INF)
    if n_valid > 0:
        dots = k[:n_valid] @ q.T                     # [n_valid, Hi]
        out[:n_valid] = np.maximum(dots, 0.0) @ ws   # weighted head sum of the ReLU
    return out


# --------------------------------------------------------------------------------------
# Step 2: top-k
# --------------------------------------------------------------------------------------
def topk_row(scores_row, n_valid, k_eff, k_base) -> np.ndarray:
    """Top-k ids of one row, as int64 [k_eff].

    K_t = min(k_eff, n_valid) columns with the largest score among j < n_valid.
    READING: ties go to the lower local index; ids are returned in ascending order,
    followed by -1 in slots K_t .. k_eff-1  ([I5776, csa.py sparse-attention excerpt]:
    picks at or beyond the causal limit become -1).
    Ids are global: cu_k[s] + local  ([PR8539, item 1]: b * S_k + local for BSHD;
    [I5776, dsa_kernels.py excerpt]: flat ids over the packed key buffer for THD).
    Plain definition: sort the visible columns by (-score, j) and keep the first K_t.
    """
    out = np.full(k_eff, -1, dtype=np.int64)
    kt = min(k_eff, n_valid)
    if kt <= 0:
        return out
    vals = np.asarray(scores_row[:n_valid], dtype=np.float64)
    cols = np.arange(n_valid)
    order = np.lexsort((cols, -vals))   # primary key: -score; secondary: column
    chosen = np.sort(order[:kt])
    out[:kt] = chosen + k_base
    return out


# --------------------------------------------------------------------------------------
# Step 3: window + top-k sparse attention with a sink
# --------------------------------------------------------------------------------------
def window_rows(t: int, q_start: int, window: int) -> np.ndarray:
    """Original-KV rows attended by query row t.  PARITY UNPINNED.

    The pages use ``window_idxs`` (concatenated before the compressed ids in the
    csa.py sparse-attention excerpt of [I5776]) without defining it.  READING: the
    `window` most recent original rows of the same segment, the query row itself
    included:  { t' : max(q_start, t - window + 1) <= t' <= t }.
    """
    lo = max(q_start, t - window + 1)
    return np.arange(lo, t + 1, dtype=np.int64) if window > 0 else np.zeros(0, dtype=np.int64)


@dataclass
class AttnRow:
    out: np.ndarray      # [H, D]
    lse: np.ndarray      # [H]   log Z_h (sink, window and selected compressed keys)
    lse_nc: np.ndarray   # [H]   u_h = log(exp(a_h) + sum_W exp(w_hr))
    cmass: np.ndarray    # [k_eff] sum_h exp(c_hj - lse_h) at valid slots, 0 at -1 slots
    c: np.ndarray        # [H, n_sel] compressed logits of the valid slots
    w: np.ndarray        # [H, n_win] window logits


def _logsumexp(x, axis=-1):
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=axis, keepdims=True) if x.shape[axis] else None
    if m is None:
        return np.full(np.delete(np.array(x.shape), axis), NEG_INF)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    s = np.sum(np.exp(x - m_safe), axis=axis, keepdims=True)
    with np.errstate(divide="ignore"):
        r = np.log(s) + m_safe
    return np.squeeze(r, axis=axis)


def attention_row(q_t, kv, ckv, sink, ids_row, win_rows, scale) -> AttnRow:
    """Sparse attention of one query row, formulation A (explicit softmax).

    [I5776, "Paper reference"]: for head h, with compressed logits c_hj, window logits
    w_hr and sink logit a_h,
        Z_h = exp(a_h) + sum_{j in C} exp(c_hj) + sum_{r in W} exp(w_hr).
    [I5776, csa.py sparse-attention excerpt]: the attention runs over the window ids
    concatenated with the selected compressed ids, with ``attn_sink`` passed as fp32
    and ``softmax_scale`` on the q.k products; -1 ids are excluded.
    READING: one KV row per position serves as both key and value and is shared by all
    heads (``compressed_kv`` expanded over heads); the sink is a raw logit (not scaled)
    that enters Z_h only and carries no value.

    The row [a_h | w_h,. | c_h,.] is soft-maxed explicitly; out is the probability-
    weighted sum of the KV rows (sink column dropped); lse_h = log Z_h; lse_nc_h is the
    log of the sink+window part; cmass_j = sum_h P_h[c column j].
    q_t: [H, D]; kv: [T, D]; ckv: [T_k, D]; sink: [H]; ids_row: [k_eff] global or -1.
    """
    q = np.asarray(q_t, dtype=np.float64)
    H, D = q.shape
    k_eff = len(ids_row)
    sel = np.array([j for j in range(k_eff) if ids_row[j] >= 0], dtype=np.int64)
    krows = np.asarray(ckv, dtype=np.float64)[np.asarray(ids_row)[sel]] if len(sel) else np.zeros((0, D))
    wrows = np.asarray(kv, dtype=np.float64)[win_rows] if len(win_rows) else np.zeros((0, D))
    c = float(scale) * (q @ krows.T)                 # [H, n_sel]
    w = float(scale) * (q @ wrows.T)                 # [H, n_win]
    a = np.asarray(sink, dtype=np.float64).reshape(H, 1)
    logits = np.concatenate([a, w, c], axis=1)       # [H, 1 + n_win + n_sel]
    lse = _logsumexp(logits, axis=1)                 # [H]
    lse_nc = _logsumexp(np.concatenate([a, w], axis=1), axis=1)
    finite = np.isfinite(lse)
    P = np.zeros_like(logits)
    P[finite] = np.exp(logits[finite] - lse[finite, None])
    vals = np.concatenate([wrows, krows], axis=0)    # value rows, sink excluded
    out = P[:, 1:] @ vals                            # [H, D]
    cm = np.zeros(k_eff)
    cm[sel] = P[:, 1 + wrows.shape[0]:].sum(axis=0)
    return AttnRow(out=out, lse=lse, lse_nc=lse_nc, cmass=cm, c=c, w=w)


def attention_row_lse_form(q_t, kv, ckv, sink, ids_row, win_rows, scale):
    """Formulation B of the same row, through the LSE decomposition of the proposal
    comment in [I5776]'s discussion thread:
        u_h   = log( exp(a_h) + sum_{r in W_valid} exp(w_hr) )
        l_h   = log( exp(u_h) + sum_{j in C} exp(c_hj) ),     p_hj = exp(c_hj - l_h)
    Returns (lse = l_h, lse_nc = u_h, p [H, n_sel], pw [H, n_win], out [H, D]) computed
    without ever forming the concatenated row; formulation A must agree with it.
    """
    q = np.asarray(q_t, dtype=np.float64)
    H, D = q.shape
    ids = np.asarray(ids_row)
    valid = ids[ids >= 0]
    krows = np.asarray(ckv, dtype=np.float64)[valid] if len(valid) else np.zeros((0, D))
    wrows = np.asarray(kv, dtype=np.float64)[win_rows] if len(win_rows) else np.zeros((0, D))
    out = np.zeros((H, D))
    lse = np.zeros(H)
    u = np.zeros(H)
    p = np.zeros((H, len(valid)))
    pw = np.zeros((H, len(win_rows)))
    for h in range(H):
        c_h = [float(scale) * float(np.dot(q[h], krows[j])) for j in range(len(valid))]
        w_h = [float(scale) * float(np.dot(q[h], wrows[r])) for r in range(len(win_rows))]
        a_h = float(sink[h])
        # u_h: log of the sink plus window mass, accumulated term by term
        terms = [a_h] + w_h
        m = max(terms)
        u_h = NEG_INF if m == NEG_INF else m + math.log(sum(math.exp(x - m) for x in terms))
        terms2 = [u_h] + c_h
        m2 = max(terms2)
        l_h = NEG_INF if m2 == NEG_INF else m2 + math.log(sum(math.exp(x - m2) for x in terms2))
        u[h], lse[h] = u_h, l_h
        if l_h == NEG_INF:
            continue
        for j, cj in enumerate(c_h):
            p[h, j] = math.exp(cj - l_h)
            out[h] += p[h, j] * krows[j]
        for r, wr in enumerate(w_h):
            pw[h, r] = math.exp(wr - l_h)
            out[h] += pw[h, r] * wrows[r]
    return lse, u, p, pw, out


# --------------------------------------------------------------------------------------
# Step 4: teacher
# --------------------------------------------------------------------------------------
def teacher_from_mass(m) -> np.ndarray:
    """t = m / max(sum m, 1e-10): the head-summed probabilities with one final L1
    normalisation over the compressed support  [I5776, "Paper reference", t_j equation;
    dsa.py excerpt: L1 normalisation with clamp(min=1e-10)]."""
    m = np.asarray(m, dtype=np.float64)
    return m / max(float(np.sum(m)), EPS_L1)


def teacher_sparse_row(attn: AttnRow, ids_row) -> np.ndarray:
    """Sparse-loss teacher over the k_eff slots of the row (0 at -1 slots).

    [I5776, proposal comment]: for the sparse loss the support C is the selected top-k
    intersected with the causally valid entries used by the core attention, and the
    per-head denominator l_h keeps the sink and window terms -- with C equal to the
    attention's compressed set, l_h is the attention's own log Z_h, so
    m_j = sum_h exp(c_hj - log Z_h) = cmass_j."""
    return teacher_from_mass(attn.cmass)


def dense_logits_row(q_t, ckv_seg, n_valid, scale) -> np.ndarray:
    """c_hj = scale * q[t,h,:] . ckv[cu_k[s] + j, :] for every causally visible key
    j < n_valid (the dense support).  Returns [H, n_valid]."""
    q = np.asarray(q_t, dtype=np.float64)
    k = np.asarray(ckv_seg, dtype=np.float64)[:n_valid]
    return float(scale) * (q @ k.T)


def teacher_dense_row(q_t, ckv_seg, n_valid, lse_nc, scale) -> np.ndarray:
    """Dense-loss teacher over j < n_valid.

    [I5776, proposal comment]: for the dense loss, C is the set of all causally visible
    compressed entries, l_h = log(exp(u_h) + sum_{j in C} exp(c_hj)) with u_h the
    sink+window log-mass of the core attention, p_hj = exp(c_hj - l_h); then the head
    sum and one L1 normalisation.  READING: u_h is the same lse_nc the sparse attention
    produces for this row (the window and sink do not depend on the loss mode)."""
    c = dense_logits_row(q_t, ckv_seg, n_valid, scale)            # [H, n_valid]
    u = np.asarray(lse_nc, dtype=np.float64).reshape(-1, 1)
    ell = _logsumexp(np.concatenate([u, c], axis=1), axis=1)      # [H]
    p = np.exp(c - ell[:, None])
    return teacher_from_mass(p.sum(axis=0))


# --------------------------------------------------------------------------------------
# Step 5: predictor, KL and the loss reduction
# --------------------------------------------------------------------------------------
def predictor(scores_vals) -> np.ndarray:
    """Softmax of the indexer scores over the support C.

    Sparse: [I5776, dsa_kernels.py excerpt] gathers the scores at the top-k ids (slots
    with id -1 get ``finfo.min`` and so zero probability) and soft-maxes them; the dsa.py
    excerpt reaches the same by adding the -inf index mask before the softmax.
    Dense: the softmax over every causally visible key (the row logsumexp)."""
    x = np.asarray(scores_vals, dtype=np.float64)
    if x.size == 0:
        return x
    return np.exp(x - _logsumexp(x))


def kl_row(teacher, pred) -> float:
    """KL(t || p) = sum_j t_j (log(t_j + 1e-10) - log(p_j + 1e-10)) over the support.

    [I5776, dsa.py excerpt]: the KL is taken with both 1e-10 epsilons as written;
    the review comment asks that the predictor-side epsilon stay log(p + 1e-10)."""
    t = np.asarray(teacher, dtype=np.float64)
    p = np.asarray(pred, dtype=np.float64)
    return float(np.sum(t * (np.log(t + EPS_LOG) - np.log(p + EPS_LOG))))


def reduce_loss(kl_rows, total_q: int, per_token: bool) -> float:
    """Loss reduction.  READING (the dsa.py excerpt is cut off before the reduction):
    per-row KL sum, then the mean over all physical query rows -- rows with nothing
    visible and padding rows contribute 0 but stay in the divisor, as the review comment
    in [I5776] describes for padded THD (real segment losses weighted by their real
    lengths, divided by the physical total_q).  With per-token loss the per-row values
    are summed."""
    s = float(np.sum(np.asarray(kl_rows, dtype=np.float64)))
    return s if per_token else s / float(total_q)


# --------------------------------------------------------------------------------------
# Whole path for a set of rows
# --------------------------------------------------------------------------------------
@dataclass
class Problem:
    """All inputs of the path as host arrays (values exactly as the GPU reads them)."""
    layout: Layout
    q: np.ndarray        # [T, H, D]
    kv: np.ndarray       # [T, D]       original KV rows (window)
    ckv: np.ndarray      # [T_k, D]     compressed KV rows
    q_idx: np.ndarray    # [T, Hi, Di]
    k_idx: np.ndarray    # [T_k, Di]
    weights: np.ndarray  # [T, Hi]      fp32
    sink: np.ndarray     # [H]          fp32
    topk: int
    window: int
    scale: float         # attention softmax scale
    idx_scale: float     # indexer softmax scale
    sparse_loss: bool = True
    per_token: bool = False


@dataclass
class RowResult:
    t: int
    geom: RowGeom
    scores: np.ndarray   # [S_k(s)] local columns, -inf where masked
    ids: np.ndarray      # [k_eff]
    attn: AttnRow
    teacher: np.ndarray  # sparse: [k_eff]; dense: [n_valid]
    pred: np.ndarray     # same support as teacher
    kl: float


def run_row(P: Problem, t: int, ids_override=None, scores_override=None) -> RowResult:
    """Every step of the path for query row t.

    ids_override / scores_override let a test run steps 3-5 on ids (or scores) that came
    from elsewhere, so later steps can be compared on identical selections."""
    L = P.layout
    g = row_geometry(L, t)
    k_eff = k_eff_of(L, P.topk)
    seg_k = slice(g.k_base, int(L.cu_k[g.seg + 1]))
    if scores_override is not None:
        scores = np.asarray(scores_override, dtype=np.float64)
    else:
        scores = indexer_scores_row(P.q_idx[t], P.weights[t], P.k_idx[seg_k], P.idx_scale, g.n_valid)
    ids = topk_row(scores, g.n_valid, k_eff, g.k_base) if ids_override is None else np.asarray(ids_override, dtype=np.int64)
    win = window_rows(t, g.q_start, P.window)
    attn = attention_row(P.q[t], P.kv, P.ckv, P.sink, ids, win, P.scale)
    if g.n_valid == 0 or g.padding:
        # no visible compressed key: the row's loss terms are zeroed
        # ([I5776, dsa.py excerpt]: fully masked rows are zeroed before and after the softmax).
        # A padding row keeps its scores, ids and attention output (the fused path masks
        # clones of them for the loss only) and contributes nothing to the loss
        # ([I5776, fused-path excerpt, steps 4b and 5]).
        n = k_eff if P.sparse_loss else 0
        return RowResult(t, g, scores, ids, attn, np.zeros(n), np.zeros(n), 0.0)
    if P.sparse_loss:
        valid = ids >= 0
        teacher = teacher_sparse_row(attn, ids)
        pred = np.zeros(k_eff)
        pred[valid] = predictor(scores[ids[valid] - g.k_base])
        kl = kl_row(teacher[valid], pred[valid])
    else:
        teacher = teacher_dense_row(P.q[t], P.ckv[seg_k], g.n_valid, attn.lse_nc, P.scale)
        pred = predictor(scores[:g.n_valid])
        kl = kl_row(teacher, pred)
    return RowResult(t, g, scores, ids, attn, teacher, pred, kl)


def run_all(P: Problem):
    """Every row, plus the reduced loss.  Only for inputs small enough for a CPU."""
    rows = [run_row(P, t) for t in range(P.layout.total_q)]
    loss = reduce_loss([r.kl for r in rows], P.layout.total_q, P.per_token)
    return rows, loss


# --------------------------------------------------------------------------------------
# Next step after the path: the indexer-loss backward
# --------------------------------------------------------------------------------------
# [I5776, proposal comment and its follow-up review]: the loss keeps a custom backward that
# recomputes what it needs from saved tensors and returns gradients only for the indexer
# q, weights and k; every teacher-side input (hence the teacher itself) is detached, and
# the top-k selection is a fixed, non-differentiable choice.  [PR8539, item 1 and test
# plan]: the sparse path's ids are global, and a batch of two rows-sets must give the
# same gradients as two single runs scaled for the row-mean loss.

def kl_grad_scores(teacher, pred) -> np.ndarray:
    """dKL/ds over the support, teacher held fixed.

    KL = sum_j t_j (log(t_j + eps) - log(p_j + eps)) with p = softmax(s):
        dKL/dp_j = -t_j / (p_j + eps),   dp_j/ds_k = p_j (delta_jk - p_k)
        => dKL/ds_k = p_k R - r_k,   r_j = t_j p_j / (p_j + eps),   R = sum_j r_j
    (with eps -> 0 this is the familiar p - t)."""
    t = np.asarray(teacher, dtype=np.float64)
    p = np.asarray(pred, dtype=np.float64)
    r = t * p / (p + EPS_LOG)
    return p * np.sum(r) - r


def indexer_grads_row(q_idx_t, w_t, k_idx_seg, idx_scale, cols, g_cols, exact_ws: bool = False):
    """Gradients of sum_c g_c * I[t, cols[c]] (I from ``indexer_scores_row``) with respect
    to q_idx[t] ([Hi, Di]), w[t] ([Hi]) and the key rows k_idx_seg[cols] ([n, Di]).

    With d_hj = q_idx[t, h] . k_j, a_hj = [d_hj > 0] and ws_h = w_h * s_idx:
        dq[h]  = ws_h * sum_j g_j a_hj k_j
        dw[h]  = s_idx * sum_j g_j max(d_hj, 0)
        dk[j]  = g_j * sum_h ws_h a_hj q[h]
    READING: the weight gradient treats ws = w * s_idx as exact (the fp32 rounding of the
    forward product has derivative 1 almost everywhere)."""
    q = np.asarray(q_idx_t, dtype=np.float64)
    cols = np.asarray(cols, dtype=np.int64)
    k = np.asarray(k_idx_seg, dtype=np.float64)[cols]
    g = np.asarray(g_cols, dtype=np.float64)
    ws = indexer_weight_scale(w_t, idx_scale, exact_ws).astype(np.float64)
    d = k @ q.T                                   # [n, Hi]
    a = (d > 0.0).astype(np.float64)
    ga = g[:, None] * a                           # [n, Hi]
    dq = ws[:, None] * (ga.T @ k)                 # [Hi, Di]
    dw = float(np.float32(idx_scale)) * (g @ np.maximum(d, 0.0))
    dk = (ga * ws[None, :]) @ q                   # [n, Di]
    return dq, dw, dk


def loss_support(P: Problem, r: RowResult):
    """The support C of row r as local columns, with the teacher and predictor on it."""
    g = r.geom
    if g.n_valid == 0 or g.padding:
        return np.zeros(0, dtype=np.int64), np.zeros(0), np.zeros(0)
    if P.sparse_loss:
        valid = r.ids >= 0
        return r.ids[valid] - g.k_base, r.teacher[valid], r.pred[valid]
    return np.arange(g.n_valid, dtype=np.int64), r.teacher, r.pred


def indexer_loss_backward(P: Problem, rows=None, grad_loss: float = 1.0):
    """dLoss/dq_idx [T, Hi, Di], dLoss/dweights [T, Hi], dLoss/dk_idx [T_k, Di] for the
    reduced loss of ``run_all`` (mean over physical rows, or the per-token sum), with the
    teacher and the selection held fixed.  rows: RowResults of every row (recomputed if
    None)."""
    L = P.layout
    T = L.total_q
    if rows is None:
        rows = [run_row(P, t) for t in range(T)]
    scale = float(grad_loss) if P.per_token else float(grad_loss) / float(T)
    dq = np.zeros(P.q_idx.shape, dtype=np.float64)
    dw = np.zeros(P.weights.shape, dtype=np.float64)
    dk = np.zeros(P.k_idx.shape, dtype=np.float64)
    for r in rows:
        cols, tch, prd = loss_support(P, r)
        if cols.size == 0:
            continue
        gs = scale * kl_grad_scores(tch, prd)
        g = r.geom
        seg_k = slice(g.k_base, int(L.cu_k[g.seg + 1]))
        dq_t, dw_t, dk_c = indexer_grads_row(P.q_idx[r.t], P.weights[r.t], P.k_idx[seg_k],
                                             P.idx_scale, cols, gs)
        dq[r.t] = dq_t
        dw[r.t] = dw_t
        np.add.at(dk, g.k_base + cols, dk_c)
    return dq, dw, dk


def indexer_loss_fixed(P: Problem, rows, q_idx=None, weights=None, k_idx=None, exact_ws: bool = True) -> float:
    """The reduced loss as a function of the indexer inputs alone: the teacher and the
    support of every row are taken from ``rows`` and held fixed, the scores recomputed
    from (q_idx, weights, k_idx).  Used to pin ``indexer_loss_backward`` by finite
    differences."""
    L = P.layout
    q_idx = P.q_idx if q_idx is None else q_idx
    weights = P.weights if weights is None else weights
    k_idx = P.k_idx if k_idx is None else k_idx
    kls = []
    for r in rows:
        cols, tch, _ = loss_support(P, r)
        if cols.size == 0:
            kls.append(0.0)
            continue
        g = r.geom
        seg_k = slice(g.k_base, int(L.cu_k[g.seg + 1]))
        sc = indexer_scores_row(q_idx[r.t], weights[r.t], k_idx[seg_k], P.idx_scale, g.n_valid, exact_ws)
        kls.append(kl_row(tch, predictor(sc[cols])))
    return reduce_loss(kls, L.total_q, P.per_token)

"""DSA hot path, float64 reference (TEST INFRASTRUCTURE ONLY).

The three stages follow the pages' formulas:

1. Lightning-indexer score.  I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s]), one
   key head shared by all indexer heads (page "arXiv'25 | DSA ... DeepSeek-V3.2",
   section 3, first equation; page "DeepSeekV3.2之DSA", part 3.1 symbol table).
   With FP8 inputs each dot product is taken over the dequantised values
   sq[t,j]*q8[t,j,:] and sk[s]*k8[s,:] (same page, part 4.3, operation order).
   No extra constant is applied: any fixed factor (n_heads^-1/2, d^-1/2) belongs
   to the caller's w (part 4.3 folds such factors into the weights).
2. Top-k.  The indices of the min(k, n) largest scores among the visible
   history (section 3, second equation; part 4.4 takes min(topk, end_pos)).
   Readings: ties go to the lower position; -0 and +0 are equal; the result is
   returned in ascending position order, padded with -1.  When n <= k every
   position is selected, i.e. the layer degrades to full attention (part 3.3 and
   part 4.5).
3. Sparse MQA-mode MLA attention over the selected latent rows (section 3,
   third equation; part 5.1: softmax(q . [c_kv; k_pe]^T) . c_kv).  The value
   is the first 512 dims of each 576-wide latent row.  An empty selection gives
   O = 0 and lse = -inf.  lse is the natural-log sum of exp of the scaled logits.

Visibility: a query sees positions [0, n_vis) of its own sequence; decode uses
n_vis = L (the whole cached history), causal prefill uses n_vis = t for query t
(strictly earlier positions, as in the TopK equation's range 1..t-1).
"""

import numpy as np

from .bf16 import bf16_decode
from .fp8 import e4m3_decode
from .layout import phys_rows

DV = 512  # value width: the latent part of each 576-wide row


# --------------------------------------------------------------------------- #
# 1. indexer
# --------------------------------------------------------------------------- #
def indexer_scores_query(q8, q_scale, w, k8, k_scale):
    """Scores of one query against n keys.

    q8 [H, D] uint8 E4M3, q_scale [H] fp32, w [H] fp32,
    k8 [n, D] uint8 E4M3, k_scale [n] fp32.
    Returns (I [n], M [n]) in float64, where M = sum_j |w_j| * ReLU(dot_j) is the
    magnitude the tolerance of the GPU comparison is taken against."""
    q = e4m3_decode(q8) * np.asarray(q_scale, np.float64)[:, None]
    k = e4m3_decode(k8) * np.asarray(k_scale, np.float64)[:, None]
    dots = q @ k.T  # [H, n]
    relu = np.maximum(dots, 0.0)
    wd = np.asarray(w, np.float64)
    return wd @ relu, np.abs(wd) @ relu


def indexer_scores(q8, q_scale, w, k8, k_scale, q_seq, q_nvis, *, row0=None,
                   block_table=None, block_size=0, queries=None):
    """Scores for a batch of queries; returns a list of float64 arrays [n_vis]
    (one per query, or per entry of ``queries`` if given)."""
    sel = range(len(q_nvis)) if queries is None else queries
    out = []
    for i in sel:
        n = int(q_nvis[i])
        rows = phys_rows(int(q_seq[i]), np.arange(n), row0=row0,
                         block_table=block_table, block_size=block_size)
        out.append(indexer_scores_query(q8[i], q_scale[i], w[i], k8[rows], k_scale[rows])[0])
    return out


# --------------------------------------------------------------------------- #
# 2. top-k
# --------------------------------------------------------------------------- #
def topk(scores, k):
    """Indices of the min(k, n) largest scores, ties to the lower index.

    Returns (idx int64 [k] ascending, padded with -1, count)."""
    v = np.asarray(scores, dtype=np.float64).copy()
    if np.isnan(v).any():
        raise ValueError("NaN scores are outside the method's domain")
    v[v == 0.0] = 0.0  # -0 -> +0: float equality already treats them as equal
    n = v.shape[0]
    count = min(int(k), n)
    order = np.lexsort((np.arange(n), -v))  # by descending score, then position
    chosen = np.sort(order[:count])
    idx = np.full(int(k), -1, dtype=np.int64)
    idx[:count] = chosen
    return idx, count


# --------------------------------------------------------------------------- #
# 3. attention
# --------------------------------------------------------------------------- #
def sparse_mla(q, kv_rows, softmax_scale, dv=DV):
    """Softmax attention of H query heads over the given latent rows.

    q [H, 576] bf16 bits, kv_rows [n, 576] bf16 bits (already gathered).
    Returns (O [H, dv], lse [H]) in float64."""
    qd = bf16_decode(q)
    h = qd.shape[0]
    kd = bf16_decode(kv_rows).reshape(-1, qd.shape[1])
    if kd.shape[0] == 0:
        return np.zeros((h, dv)), np.full(h, -np.inf)
    z = float(softmax_scale) * (qd @ kd.T)  # [H, n]
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ kd[:, :dv]) / l
    return o, (m + np.log(l))[:, 0]


def dense_mla(q, kv_history, softmax_scale, dv=DV):
    """Full attention over the whole visible history, written head by head with
    a log-sum-exp reduction (a separate formulation used to check that the
    sparse path degrades to full attention when the history fits in k)."""
    qd = bf16_decode(q)
    kd = bf16_decode(kv_history).reshape(-1, qd.shape[1])
    h = qd.shape[0]
    o = np.zeros((h, dv))
    lse = np.full(h, -np.inf)
    for i in range(h):
        if kd.shape[0] == 0:
            continue
        logits = float(softmax_scale) * (kd @ qd[i])
        lse[i] = np.logaddexp.reduce(logits)
        o[i] = np.exp(logits - lse[i]) @ kd[:, :dv]
    return o, lse


# --------------------------------------------------------------------------- #
# composition
# --------------------------------------------------------------------------- #
def forward_query(q8, q_scale, w, k8_hist, k_scale_hist, q_mla, kv_hist, k,
                  softmax_scale):
    """One query through indexer -> top-k -> sparse attention.

    ``*_hist`` hold the query's visible history in position order.
    Returns (O, lse, idx, count, scores); with n_vis <= k the indexer is skipped
    and every position is attended."""
    n = kv_hist.shape[0]
    if n <= k:
        idx = np.full(int(k), -1, dtype=np.int64)
        idx[:n] = np.arange(n)
        scores = None
        count = n
    else:
        scores, _ = indexer_scores_query(q8, q_scale, w, k8_hist, k_scale_hist)
        idx, count = topk(scores, k)
    o, lse = sparse_mla(q_mla, kv_hist[idx[:count]], softmax_scale)
    return o, lse, idx, count, scores

"""Indexer alignment loss and its gradients, float64 (TEST INFRASTRUCTURE ONLY).

Training the lightning indexer (page "arXiv'25 | DSA ... DeepSeek-V3.2",
sections 5.1 and 5.2, the two L_I equations; the mlpod.com page on
DeepSeek-V3.2-Exp, parts 2.1.1 and 2.1.2):

* Target.  For query t, the main attention's distribution of every head over
  the attended positions is summed over the heads, and the sum is L1-normalised
  along the positions: p[t,:].  Reading: "attention scores" are the softmax
  probabilities (the logits can be negative, and only probabilities make an L1
  normalisation a distribution).  The attention is the MQA-mode MLA of the
  forward pass: logits z[h,s] = softmax_scale * q[h,:] . kv[s,:] over the
  576-wide latent rows.
* Loss.  L_I = sum_t KL(p[t,:] || Softmax(I[t,:])), the softmax taken over the
  same positions as the target.  Dense warm-up: every visible position.  Sparse
  stage: only the selected set S_t, where the attention itself runs over S_t,
  so the target is the head-summed attention over S_t, L1-normalised over S_t.
  Terms with p = 0 contribute 0 (the usual 0 log 0 = 0 convention).
* Gradient.  Only the indexer learns from L_I, and its inputs are detached
  from the main model, so the target p is a constant: dL/dI[t,s] =
  Softmax(I[t,:])[s] * sum(p[t,:]) - p[t,s] (= Softmax - p, since p sums to 1).
  Through the indexer score I[t,s] = sum_j w[t,j] * ReLU(qh[t,j,:] . kh[s,:])
  (qh, kh the dequantised FP8 query and key; page "arXiv'25 | DSA ...",
  section 3, first equation): dw, dqh and dkh below.  Reading: the derivative
  of ReLU at exactly 0 is taken as 0, and the FP8 quantiser is passed through
  unchanged (gradients are with respect to the dequantised values).
"""

import numpy as np

from .bf16 import bf16_decode
from .fp8 import e4m3_decode


def attention_target(q, kv_rows, softmax_scale):
    """Head-summed, L1-normalised attention distribution over the given rows.

    q [H, 576] bf16 bits; kv_rows [n, 576] bf16 bits (the attended rows, in set
    order).  Returns p [n] float64 (empty for n = 0)."""
    qd = bf16_decode(q)
    kd = bf16_decode(kv_rows).reshape(-1, qd.shape[1])
    if kd.shape[0] == 0:
        return np.zeros(0)
    z = float(softmax_scale) * (qd @ kd.T)  # [H, n]
    e = np.exp(z - z.max(axis=1, keepdims=True))
    probs = e / e.sum(axis=1, keepdims=True)  # each head's softmax over the rows
    a = probs.sum(axis=0)  # summed over the heads
    return a / np.abs(a).sum()  # L1 normalisation along the positions


def kl_to_softmax(p, logits):
    """KL(p || Softmax(logits)) and its gradient with respect to the logits.

    Returns (kl, grad [n], mag) where mag = sum_s |p_s (ln p_s - ln q_s)|, the
    magnitude of the sum (the scale a GPU result is compared against)."""
    p = np.asarray(p, dtype=np.float64)
    x = np.asarray(logits, dtype=np.float64)
    if x.shape[0] == 0:
        return 0.0, np.zeros(0), 0.0
    m = x.max()
    log_q = x - m - np.log(np.exp(x - m).sum())
    terms = np.zeros_like(p)
    pos = p > 0
    terms[pos] = p[pos] * (np.log(p[pos]) - log_q[pos])
    grad = np.exp(log_q) * p.sum() - p
    return float(terms.sum()), grad, float(np.abs(terms).sum())


def indexer_kl_query(q, kv_rows, scores, softmax_scale):
    """One query's loss term over its attended set.

    kv_rows [n, 576] bf16 bits and scores [n] (the indexer's I at the same
    positions, in the same order).  Returns (kl, grad [n], p [n], mag)."""
    p = attention_target(q, kv_rows, softmax_scale)
    kl, grad, mag = kl_to_softmax(p, scores)
    return kl, grad, p, mag


def indexer_logits(qh, w, kh):
    """I[s] = sum_j w_j * ReLU(qh_j . kh_s) on real-valued (dequantised) inputs:
    qh [H_I, d], w [H_I], kh [n, d] -> [n] float64."""
    dots = np.asarray(qh, np.float64) @ np.asarray(kh, np.float64).T
    return np.asarray(w, np.float64) @ np.maximum(dots, 0.0)


def dequantise(codes, scales):
    """FP8 E4M3 codes [n, d] times per-row scales [n] -> float64 [n, d]."""
    return e4m3_decode(codes) * np.asarray(scales, np.float64)[:, None]


def indexer_backward_query(qh, w, kh, g):
    """Gradients of sum_s g[s] * I[s] with respect to the indexer's inputs.

    qh [H_I, d], w [H_I], kh [n, d] (dequantised), g [n] = dL/dI over the set.
    Returns (dw [H_I], dqh [H_I, d], dkh [n, d]) in float64:
      dw[j]     = sum_s g[s] ReLU(qh_j . kh_s)
      dqh[j,:]  = w[j] sum_s g[s] [qh_j . kh_s > 0] kh_s
      dkh[s,:]  = g[s] sum_j w[j] [qh_j . kh_s > 0] qh_j
    """
    qh = np.asarray(qh, np.float64)
    kh = np.asarray(kh, np.float64)
    w = np.asarray(w, np.float64)
    g = np.asarray(g, np.float64)
    dots = qh @ kh.T  # [H_I, n]
    active = dots > 0.0
    dw = np.maximum(dots, 0.0) @ g
    gate = active * (w[:, None] * g[None, :])  # dI[s] / d(dot[j, s]) times g[s]
    return dw, gate @ kh, gate.T @ qh

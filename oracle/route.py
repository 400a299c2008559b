"""Router logits, top-k selection and routing weights (oracle; test infrastructure only).

ExactMoE (page "Every Expert Counts: ExactMoE for Memory-Efficient W4A16
Inference", Abstract) keeps the router in BF16 and leaves the top-k routing
procedure unchanged.  Readings taken where the page is silent:

* logits l[t, e] = sum_c x[t, c] * Wr[e, c] over bf16 inputs and bf16 router
  weights.  The products are exact; the sum is formed in float64 and the logit
  is then rounded once to float32, the precision in which the selection is
  made on both sides;
* selection orders experts by (logit descending, expert index ascending) and
  keeps the first k, emitted in that order (ties go to the lower index);
* weights: softmax over the selected logits, w_j = exp(l_j - l_max) /
  sum_{i in top-k} exp(l_i - l_max), which equals the softmax over all E
  renormalised over the top-k (renormalize=True, the default, so each token's
  weights sum to 1).  With renormalize=False the denominator runs over all E.
"""
import numpy as np

from . import bf16


def logits_f64(x_bits, wr_bits):
    """float64 logits [T, E] = x @ Wr^T from bf16 bit patterns x [T, d], Wr [E, d]."""
    return bf16.to_f64(x_bits) @ bf16.to_f64(wr_bits).T


def logits_f32(x_bits, wr_bits):
    """Logits rounded once to float32 (the precision the selection is made in)."""
    return logits_f64(x_bits, wr_bits).astype(np.float32)


def topk_select(logits, k):
    """Indices [T, k] of the k largest logits per row, ties to the lower index, largest first."""
    logits = np.asarray(logits)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    idx = np.arange(E)
    for t in range(T):
        order = np.lexsort((idx, -logits[t].astype(np.float64)))   # primary: -logit, then index
        ids[t] = order[:k]
    return ids


def topk_weights(logits, ids, renormalize=True):
    """Routing weights [T, k] (float64) for the selected ids."""
    l = np.asarray(logits, dtype=np.float64)
    sel = np.take_along_axis(l, ids.astype(np.int64), axis=1)
    lmax = np.max(l, axis=1, keepdims=True)
    num = np.exp(sel - lmax)
    den = num.sum(axis=1, keepdims=True) if renormalize else np.exp(l - lmax).sum(axis=1, keepdims=True)
    return num / den


def route(x_bits, wr_bits, k, renormalize=True):
    """(logits float32 [T, E], ids int32 [T, k], weights float64 [T, k])."""
    l32 = logits_f32(x_bits, wr_bits)
    ids = topk_select(l32, k)
    return l32, ids, topk_weights(l32, ids, renormalize)

"""Single-query attention in float64: the dense definition and the online
(block-by-block) recurrence.

Sources:
  * "Serving Language Models Within a Memory Budget", section 6: dense
    attention forms scaled query-key scores, applies softmax and multiplies by
    the values; the result is exact as an operation, not bitwise across
    evaluation orders, and extreme logits must not overflow.
  * same page, eq. (4): processing a new block of scores s_j updates the
    running maximum m' = max(m, max_j s_j) and the running normaliser
    l' = exp(m - m') l + sum_j exp(s_j - m'); the weighted-value accumulator
    is rescaled by the same factor exp(m - m').
  * "vLLM PagedAttention and continuous batching", section "PagedAttention:
    fixed blocks, non-contiguous physical memory": paging keeps the attention
    formula and only changes where keys and values are stored, so the paged
    result is the dense result over the gathered keys and values.
  * "PagedAttention and Online Inference", section 1: grouped-query attention
    changes the number of key/value heads.  Reading taken here: query head h
    uses key/value head floor(h / G) with G = H_q / H_kv (consecutive query
    heads share one key/value head).
"""

from __future__ import annotations

import numpy as np


def softmax_weights(scores: np.ndarray) -> np.ndarray:
    """Max-subtracted softmax of a 1-D float64 score vector."""
    s = np.asarray(scores, dtype=np.float64)
    if s.size == 0:
        return s.copy()
    e = np.exp(s - np.max(s))
    return e / np.sum(e)


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    if Hq % Hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    return h // (Hq // Hkv)


def dense_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """One query token per head against n contiguous keys/values.

    q: [Hq][d]  K, V: [n][Hkv][d]  (float64)  ->  out [Hq][d] float64.
    With n == 0 the output is zero (empty weighted sum).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hq, d = q.shape
    n, Hkv, _ = K.shape
    out = np.zeros((Hq, d), dtype=np.float64)
    if n == 0:
        return out
    for h in range(Hq):
        k = kv_head_of(h, Hq, Hkv)
        scores = float(scale) * (K[:, k, :] @ q[h])          # [n]
        p = softmax_weights(scores)                          # [n]
        out[h] = p @ V[:, k, :]                              # [d]
    return out


def online_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                     block: int) -> np.ndarray:
    """Same result as ``dense_attention`` by the eq. (4) recurrence over
    consecutive blocks of ``block`` keys, in float64."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hq, d = q.shape
    n, Hkv, _ = K.shape
    out = np.zeros((Hq, d), dtype=np.float64)
    for h in range(Hq):
        k = kv_head_of(h, Hq, Hkv)
        m = -np.inf          # running maximum
        ell = 0.0            # running normaliser
        acc = np.zeros(d)    # running weighted sum of values
        for start in range(0, n, block):
            s = float(scale) * (K[start:start + block, k, :] @ q[h])
            m_new = max(m, float(np.max(s)))
            factor = np.exp(m - m_new)          # exp(-inf) = 0 on the first block
            w = np.exp(s - m_new)
            ell = factor * ell + float(np.sum(w))
            acc = factor * acc + w @ V[start:start + block, k, :]
            m = m_new
        if n:
            out[h] = acc / ell
    return out
